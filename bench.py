#!/usr/bin/env python3
"""Benchmark of the varlen chunked Gated Delta Rule prefill on one MI355X.

A step is one full ``gdn_prefill`` call (chunk-index build where the batch
needs it, intra-chunk pass, state pass with the output, all heads) over one
batch of seeded synthetic input already resident in HBM; outputs and
workspace are allocated once.  The default workload is the GVA batch: 8
sequences of seeded lengths in [1, 8192] (23,060 tokens), 16 q/k heads and 32
v heads, head size 128, bf16 q/k/v with in-kernel q/k L2 normalisation,
checkpoints every 1024 tokens and fp32 final states.  Beside it the same run
times the 2 x 2048-token, 16-head batch (the shape of gitcode "FlashInfer GDN
Prefill 完全指南", section "基础用法") and reports it under
``"varlen_2x2048"``.

The roofline fraction uses the method's own HBM bytes: q, k, v read and o
written in the input dtype (shared q/k/v heads counted once per source head),
g and beta in fp32, plus the initial, final and checkpoint states the call
reads and writes.  The kernels' own bytes (intermediates included) are
reported beside it as ``implementation_bytes_per_launch``.

Prints one JSON line with the throughput (tokens/s over all heads, from K
steps timed with nothing else in them), the roofline position of the
dominant kernel (timed live with HIP events recorded around it on the call's
stream, in K further steps) and the CPU oracle's throughput on the same
workload (a bounded number of repetitions on this host's cores).

    python bench.py [--steps K] [--warmup W] [--workload gva8]
    python bench.py --workload decode       # the decode step, its own line
    python bench.py --copy-calibration      # plain 1 GiB copies, for counters
    python bench.py --summarize <workload> <rocprofv3 output dirs...> <command>
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 matrix peak
PHASES = ["chunk_index", "intra", "state", "output"]
DEFAULT_WORKLOAD = "gva8"
TRAFFIC_SOURCE = ("committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/traffic.json), "
                  "taken on the same kernel source (hash-matched); not measured in this run")
KERNEL_SOURCES = {
    "chunk_index": ("k0_chunk_index.hip",), "intra": ("k1_intra.hip",),
    "state": ("k2_state.hip", "k5_cp.hip"), "output": ("k3_output.hip",),
    "decode": ("k4_decode.hip",),
}
# headers every kernel source includes
COMMON_SOURCES = ("gdn_common.h", "gdn_internal.h", "gdn_state.h")


def per_token_head_bytes(wl, phase, tform=False):
    """Algorithmic HBM bytes per (token, sab head) of each phase (fp32 gates,
    q/k/v/o and intermediates in the compute dtype of width e).

    16-bit inputs (the state pass forms the output itself), W form:
      intra : reads q, k, v, g, beta; writes W and U (64 x D each per
              chunk-head), the normalised k and q fragments (64 x D per chunk
              and k / q head), the six unmasked 16 x 32 blocks of the masked
              Q K^T (48 of 64 elements per row) and the 64 cumulative log
              gates
      state : reads W, the k fragments, U, the q fragments, those Q K^T
              blocks and the gates; writes o
    16-bit inputs, T form (tform):
      intra : reads q, k, g, beta; writes -T diag(beta) (64 x 64 per
              chunk-head), the q fragments, the Q K^T blocks, the gates and
              two rows of scales
      state : reads k, v, -T diag(beta), the q fragments, the Q K^T blocks,
              the gates and the scales; writes o
    fp32 inputs (separate output pass):
      intra : reads k, v, g, beta; writes W, Ktilde, U and the gates
      state : reads W, Ktilde, U, G_last; writes the chunk-start state
              (D x D per chunk-head) and the new values N (64 x D)
      output: reads q, k, chunk-start state, N, G; writes o
    Shared q/k/v heads are counted once per source head.
    """
    D, H = wl.D, wl.H
    e = 4 if wl.dtype == "f32" else 2
    hq, hk, hv = wl.q.shape[1], wl.k.shape[1], wl.v.shape[1]
    qf, kf, vf = hq / H, hk / H, hv / H
    if wl.dtype != "f32" and tform:
        inter = 64 * e + qf * D * e + 48 * e + 4 + 8
        if phase == "intra":
            return (qf + kf) * D * e + 8 + inter
        if phase == "state":
            return inter + (kf + vf) * D * e + D * e
        return 0.0
    if wl.dtype != "f32":
        inter = (2 + kf + qf) * D * e + 48 * e + 4
        if phase == "intra":
            return (qf + kf + vf) * D * e + 8 + inter
        if phase == "state":
            return inter + D * e
        return 0.0
    st = D * D * e / 64.0          # chunk-start state per token
    if phase == "intra":
        return (kf + vf) * D * e + 8 + 3 * D * e + 4
    if phase == "state":
        return 3 * D * e + 4.0 / 64 + st + D * e
    if phase == "output":
        return (qf + kf) * D * e + st + D * e + 4 + D * e
    return 0.0


STATE_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1, "e5m2": 1}


def method_bytes(wl):
    """The method's HBM bytes for one call, independent of how the kernels
    split the work: per (token, sab head) q, k and v read and o written in
    the input dtype (shared heads counted once per source head) and g, beta
    in fp32 -- 1,032 B with equal heads at D = 128 in bf16, 776 B with 16
    q/k heads and 32 v heads -- plus, per (sequence, head), the initial state
    read, the final state written and every checkpoint row written."""
    D, H, T, N = wl.D, wl.H, wl.T, wl.N
    e = 4 if wl.dtype == "f32" else 2
    hq, hk, hv = wl.q.shape[1], wl.k.shape[1], wl.v.shape[1]
    per_th = (hq + hk + hv) / H * D * e + D * e + (8 if wl.g is not None else 0)
    total = per_th * T * H
    st = D * D * H
    if wl.initial_state is not None:
        total += N * st * STATE_BYTES[wl.initial_state_dtype]
    if wl.output_final_state:
        total += N * st * STATE_BYTES[wl.final_state_dtype]
    if wl.checkpoint_every > 0 and wl.checkpoint_cu_starts is not None:
        total += int(wl.checkpoint_cu_starts[-1]) * st * STATE_BYTES[wl.checkpoint_dtype]
    return float(total)


def cpu_model():
    """The host CPU's model name (lscpu's "Model name", from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


FLOPS_PER_TOKEN_HEAD = lambda D: 2 * (5 * 64 * D + 3 * D * D)   # eight chunk GEMMs
# the same with the five products that involve a 64 x 64 triangle (K K^T,
# Q K^T, T (beta gamma K), T (beta V), P N) counted at half a tile
FLOPS_TRI_PER_TOKEN_HEAD = lambda D: 2 * (5 * 32 * D + 3 * D * D)


def decode_bytes_per_seq_head(wl):
    """Algorithmic HBM bytes of one decode step per (sequence, sab head):
    the D x D state read and written in its pool dtype, q, k, v (shared
    heads counted once per source head), g and beta read, o written."""
    D, H = wl.D, wl.H
    e = 4 if wl.dtype == "f32" else 2
    se = {"f32": 4, "bf16": 2, "f16": 2}[wl.initial_state_dtype]
    hq, hk, hv = wl.q.shape[1], wl.k.shape[1], wl.v.shape[1]
    return 2 * D * D * se + (hq + hk + hv) / H * D * e + 8 + D * e


def hip():
    L = ctypes.CDLL("libamdhip64.so.7")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                      ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


def new_event(L):
    ev = ctypes.c_void_p()
    if L.hipEventCreate(ctypes.byref(ev)) != 0:
        raise RuntimeError("hipEventCreate failed")
    return ev


def elapsed_ms(L, a, b):
    ms = ctypes.c_float()
    if L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return float(ms.value)


def source_hash(names):
    """Hash of a phase's kernel sources and the shared headers: counters taken
    on other sources are not used."""
    d = os.path.join(ROOT, "gated_deltanet_chunked_varlen_amd", "csrc")
    h = hashlib.sha256()
    for n in tuple(names) + COMMON_SOURCES:
        with open(os.path.join(d, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(phase, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        db = json.load(f)
    rec = db.get("%s/%s" % (phase, workload))
    if not rec or rec.get("source_hash") != source_hash(KERNEL_SOURCES[phase]):
        return None
    return rec.get("bytes_per_launch")


def load_mfma(workload):
    """rocprofv3-measured matrix-core use per phase from the committed counter
    summary (profiles/mfma.json), for phases whose kernel source is
    unchanged since the counters were taken; {} if none."""
    path = os.path.join(ROOT, "profiles", "mfma.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        db = json.load(f)
    res = {}
    for ph in PHASES:
        rec = db.get("%s/%s" % (ph, workload))
        if rec and rec.get("source_hash") == source_hash(KERNEL_SOURCES[ph]):
            res[ph] = {"mfma_busy_frac": rec["mfma_busy_frac"],
                       "bf16_tflop_per_launch": rec["bf16_flop_per_launch"] / 1e12}
    return res


def cpu_baseline(wl, seconds):
    """The oracle as it stands, timed on this host: the whole workload,
    repeated until ``seconds`` have passed (at least once)."""
    from oracle import oracle
    from tests import gdn_testlib as tl
    prob = tl.oracle_problem(wl)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.token(prob)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    items = wl.N * wl.H
    return {"value": wl.T * reps / dt, "unit": "tokens/s",
            "cores": min(oracle.num_threads(), items), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "whole workload (%d tokens x %d heads), fp64 token "
                      "recurrence, %d repetition(s) in %.1f s" % (
                          wl.T, wl.H, reps, dt)}


def copy_calibration(nbytes=1 << 30, reps=5):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


PROF_KERNELS = {"chunk_index": ("chunk_index_kernel",),
                "intra": ("intra_kernel", "intra_kernel_h", "intra_tform_shared_kernel"),
                "state": ("state_kernel", "state_output_kernel", "cp_transition_kernel",
                          "cp_fixup_kernel"),
                "output": ("output_kernel",), "decode": ("decode_kernel",)}


def _phase_of(kernel_name):
    """Phase of a kernel from its (demangled) name: the bare function name is
    the identifier just before the template arguments or parameter list."""
    import re
    if kernel_name.startswith("_ZN"):          # mangled: last name of the nested name
        pos, parts = 3, []
        while pos < len(kernel_name) and kernel_name[pos].isdigit():
            m = re.match(r"\d+", kernel_name[pos:])
            n = int(m.group(0))
            pos += len(m.group(0))
            parts.append(kernel_name[pos:pos + n])
            pos += n
        base = parts[-1] if parts else kernel_name
    else:
        m = re.search(r"(\w+)\s*[<(]", kernel_name)
        base = m.group(1) if m else kernel_name
    for ph, names in PROF_KERNELS.items():
        if base in names:
            return ph
    return None


def _one(d, pat):
    import glob
    hits = glob.glob(os.path.join(d, "**", pat), recursive=True)
    if not hits:
        raise SystemExit("no %s under %s" % (pat, d))
    return hits[0]


def _counters(d):
    import collections
    import csv
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(d, "*counter_collection.csv"))):
        out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return out


def _by_phase(table):
    """Per call and phase: each kernel's mean over its dispatches, summed over
    the kernels of the phase (the context-parallel state phase runs three)."""
    res = {}
    for ph in PROF_KERNELS:
        means = [sum(vs) / len(vs) for name, vs in table.items() if _phase_of(name) == ph and vs]
        if means:
            res[ph] = sum(means)
    return res


def summarize(argv):
    """Write profiles/<workload>_kernels.md and update profiles/traffic.json
    from rocprofv3 CSV output: argv = workload, kernel-trace dir, FETCH_SIZE
    dir, WRITE_SIZE dir, copy FETCH dir, copy WRITE dir, command text.
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counters read for the plain 1 GiB copy of --copy-calibration."""
    import collections
    import csv
    import glob
    wname, kdir, fdir, wdir, cfdir, cwdir = argv[:6]
    cmd = " ".join(argv[6:])
    stats = list(csv.DictReader(open(_one(kdir, "*kernel_stats.csv"))))
    fetch, write = _by_phase(_counters(fdir)), _by_phase(_counters(wdir))
    cal_bytes = 1 << 30
    cf = [v for n, vs in _counters(cfdir).items() if "copyBuffer" in n for v in vs]
    cw = [v for n, vs in _counters(cwdir).items() if "copyBuffer" in n for v in vs]
    f_scale = cal_bytes / (sum(cf) / len(cf) * 1024.0)
    w_scale = cal_bytes / (sum(cw) / len(cw) * 1024.0)
    lines = ["# Kernel trace and HBM counters: %s" % wname, "",
             "Command (kernel trace):", "", "    " + cmd, "",
             "| kernel | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %s%% |" % (
            r["Name"][:60], r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
    lines += ["", "Counter passes: the same bench command with fewer steps under "
              "`timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` "
              "(one counter per pass).",
              "Calibration (`bench.py --copy-calibration`, 1 GiB copy): FETCH_SIZE "
              "reads %.1f KiB -> scale %.4f; WRITE_SIZE reads %.1f KiB -> scale %.4f." % (
                  sum(cf) / len(cf), f_scale, sum(cw) / len(cw), w_scale), "",
              "| kernel | FETCH KiB | WRITE KiB | HBM bytes/launch (scaled) |",
              "|---|---|---|---|"]
    db_path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(db_path)) if os.path.exists(db_path) else {}
    for ph in PROF_KERNELS:
        if ph in fetch and ph in write:
            b = fetch[ph] * 1024 * f_scale + write[ph] * 1024 * w_scale
            lines.append("| %s | %.1f | %.1f | %.4g |" % (ph, fetch[ph], write[ph], b))
            db["%s/%s" % (ph, wname)] = {
                "bytes_per_launch": b, "fetch_kib": fetch[ph], "write_kib": write[ph],
                "fetch_scale": f_scale, "write_scale": w_scale,
                "source_hash": source_hash(KERNEL_SOURCES[ph])}
    json.dump(db, open(db_path, "w"), indent=1, sort_keys=True)
    out = os.path.join(ROOT, "profiles", "%s_kernels.md" % wname)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_mfma(argv):
    """Write profiles/<workload>_mfma.md and update profiles/mfma.json from a
    rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
    SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_BUSY_CU_CYCLES: argv = workload,
    counter dir, command text.  Matrix-core busy fraction = busy cycles summed
    over the SIMDs / (GPU-active cycles of one XCD x 1024 SIMDs), the form of
    rocprofv3's own MfmaUtil metric; GRBM_GUI_ACTIVE arrives summed over the 8
    XCDs.  Executed bf16/fp16 matrix FLOP = MOPS x 512."""
    import collections
    import csv
    wname, cdir = argv[:2]
    cmd = " ".join(argv[2:])
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(_one(cdir, "*counter_collection.csv"))):
        ph = _phase_of(r["Kernel_Name"])
        if ph:
            per[ph][r["Counter_Name"]].append(float(r["Counter_Value"]))
    avg = lambda v: sum(v) / len(v)
    lines = ["# Matrix-core counters: %s" % wname, "",
             "Command:", "", "    " + cmd, "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
             "executed matrix FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (fp16 and fp32 inputs "
             "count under F16 / F32 and read 0 here). Counter runs serialise and lengthen kernels, so the "
             "busy fraction is a lower bound on the unprofiled one.", "",
             "| kernel | dispatches | MFMA busy | executed matrix GFLOP per launch |",
             "|---|---|---|---|"]
    db_path = os.path.join(ROOT, "profiles", "mfma.json")
    db = json.load(open(db_path)) if os.path.exists(db_path) else {}
    for ph in PHASES + ["decode"]:
        c = per.get(ph)
        if not c or "SQ_VALU_MFMA_BUSY_CYCLES" not in c or "GRBM_GUI_ACTIVE" not in c:
            continue
        busy = avg(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / (avg(c["GRBM_GUI_ACTIVE"]) / 8.0 * 1024.0)
        flop = avg(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0.0])) * 512.0
        lines.append("| %s | %d | %.2f%% | %.3f |" % (
            ph, len(c["SQ_VALU_MFMA_BUSY_CYCLES"]), 100.0 * busy, flop / 1e9))
        db["%s/%s" % (ph, wname)] = {"mfma_busy_frac": busy, "bf16_flop_per_launch": flop,
                                     "source_hash": source_hash(KERNEL_SOURCES[ph])}
    json.dump(db, open(db_path, "w"), indent=1, sort_keys=True)
    out = os.path.join(ROOT, "profiles", "%s_mfma.md" % wname)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def bench_decode(args):
    """The decode step on the decode workload: one JSON line of its own."""
    import torch
    from gated_deltanet_chunked_varlen_amd import workloads as W
    from gated_deltanet_chunked_varlen_amd import api
    from gated_deltanet_chunked_varlen_amd import _native as nat

    wl = W.WORKLOADS["decode"]()
    d = W.to_device(wl)
    N, H, D = wl.N, wl.H, wl.D
    pool = d["initial_state"]
    p, out, outst = api.make_params(
        d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], scale=wl.scale,
        initial_state=pool, output_final_state=True,
        use_qk_l2norm_in_kernel=wl.l2norm_in_kernel, output_state=pool,
        state_indices=d["state_indices"], decode=True)
    lib = nat.lib()
    L = hip()
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        rc = lib.gdn_decode(ctypes.byref(p), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(nat.status_string(rc))

    for _ in range(max(args.warmup, 1)):
        call()
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    # the decode step is one kernel: HIP events on the call's stream around
    # it, after untimed calls so that the clock has settled again
    pairs = [(new_event(L), new_event(L)) for _ in range(K)]
    rec = L.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    for _ in range(min(max(args.warmup, 1), 200)):
        call()
    for a_, b_ in pairs:
        if rec(a_, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        call()
        if rec(b_, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
    torch.cuda.synchronize()
    dom_ms = sum(elapsed_ms(L, a_, b_) for a_, b_ in pairs) / K
    for a_, b_ in pairs:
        L.hipEventDestroy(a_)
        L.hipEventDestroy(b_)
    bytes_launch = decode_bytes_per_seq_head(wl) * N * H
    achieved = bytes_launch / (dom_ms / 1e3) / 1e9
    res = {
        "metric": "GDN decode tokens/s (one new token per sequence per step), H=16 D=128",
        "value": N * K / (ms_total / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_total / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded numpy draws, see workloads.py)",
        "config": {"workload": wl.name, "num_seqs": N, "tokens_per_seq": 1,
                   "num_heads": H, "head_size": D, "state_pool_rows": int(pool.shape[0]),
                   "state_dtype": wl.initial_state_dtype, "qk_l2norm_in_kernel": wl.l2norm_in_kernel,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic("decode", wl.name), "avg_launch_ms": dom_ms,
                     "timing": "HIP events around the call in each of K further steps",
                     "algorithmic_bytes_per_launch": bytes_launch},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def measure_prefill(wl, steps, warmup, cold_calls, use_cp="auto"):
    """Time one prefill workload: throughput over exactly ``steps`` calls after
    ``warmup`` untimed ones, per-phase times, the dominant kernel timed with
    HIP events on the call's stream, optionally cold-cache calls.  Returns a
    dict of the raw figures."""
    import torch
    from gated_deltanet_chunked_varlen_amd import workloads as W
    from gated_deltanet_chunked_varlen_amd import api
    from gated_deltanet_chunked_varlen_amd import _native as nat

    d = W.to_device(wl)
    H, D, N, T = wl.H, wl.D, wl.N, wl.T
    kw = dict(g=d["g"], beta=d["beta"], scale=wl.scale, cu_seqlens=d["cu_seqlens"],
              use_qk_l2norm_in_kernel=wl.l2norm_in_kernel,
              output_final_state=wl.output_final_state)
    if wl.state_indices is not None:
        kw.update(initial_state=d["initial_state"], state_indices=d["state_indices"],
                  output_state=d["initial_state"])
    else:
        kw.update(initial_state=d["initial_state"])
    if wl.checkpoint_every > 0:
        rows = int(wl.checkpoint_cu_starts[-1])
        kw.update(state_checkpoints=torch.empty((rows, H, D, D), device="cuda"),
                  checkpoint_cu_starts=d["checkpoint_cu_starts"],
                  checkpoint_every_n_tokens=wl.checkpoint_every)
    p, out, outst = api.make_params(d["q"], d["k"], d["v"], use_cp=use_cp, **kw)
    need = api.workspace_size(p)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p.workspace, p.workspace_bytes = ctypes.c_void_p(ws.data_ptr()), need
    form = state_form(wl, need != api.workspace_size(api.make_params(
        d["q"], d["k"], d["v"], use_cp=False, **kw)[0]))
    lib = nat.lib()
    L = hip()
    stream = torch.cuda.current_stream().cuda_stream
    none5 = (ctypes.c_void_p * 5)()

    def call(evs=none5):
        rc = lib.gdn_prefill_timed(ctypes.byref(p), ctypes.c_void_p(stream), evs)
        if rc != 0:
            raise RuntimeError(nat.status_string(rc))

    # warm-up: W calls, the last ones with every phase timed (to find the
    # dominant kernel afterwards).  The timed region follows at once: after a
    # few ms of idleness the GPU clock drops and needs ~10 ms of work to come
    # back, so nothing (no event reads) may sit between the two.
    W_ = max(warmup, 1)
    n_ev = min(W_, 50)
    ev = [[new_event(L) for _ in range(5)] for _ in range(n_ev)]
    for i in range(W_):
        j = i - (W_ - n_ev)
        call((ctypes.c_void_p * 5)(*ev[j]) if j >= 0 else none5)

    # timed region: exactly K steps, each the call as a user makes it
    K = steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        call()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(stop)

    # median over the timed warm-up calls (after the very first call, which
    # pays one-time set-up)
    used = ev[1:] if (len(ev) > 1 and n_ev == W_) else ev
    phase_ms = {ph: float(np.median([elapsed_ms(L, e[j], e[j + 1]) for e in used]))
                for j, ph in enumerate(PHASES)}
    dom = max(PHASES, key=lambda ph: phase_ms[ph])
    di = PHASES.index(dom)

    # roofline region: K more steps with HIP events recorded on the call's own
    # stream around the dominant kernel of every step.  The two extra events
    # per step lengthen each step a little, so they stay out of the region
    # that gives the throughput.
    # It is preceded by untimed calls, so that it too runs on a settled clock.
    pairs = [(new_event(L), new_event(L)) for _ in range(K)]
    e5s = []
    for i in range(K):
        e5 = (ctypes.c_void_p * 5)()
        e5[di], e5[di + 1] = pairs[i][0], pairs[i][1]
        e5s.append(e5)
    for i in range(min(W_, 200)):
        call()
    for i in range(K):
        call(e5s[i])
    torch.cuda.synchronize()
    dom_ms = sum(elapsed_ms(L, a, b) for a, b in pairs) / K
    for row in ev:
        for e in row:
            L.hipEventDestroy(e)
    for a, b in pairs:
        L.hipEventDestroy(a)
        L.hipEventDestroy(b)

    # cold last-level cache, beside the warm steady state above: before each
    # of a few calls, 512 MiB (twice the 256 MB last-level cache) are read on
    # the call's stream (a read leaves no dirty lines to drain during the
    # call, as a write would), and the call alone is timed between the first
    # and last of its phase events
    cold = None
    if cold_calls > 0:
        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        ce = [(new_event(L), new_event(L)) for _ in range(cold_calls)]
        for i in range(cold_calls):
            flush.sum()
            e5 = (ctypes.c_void_p * 5)()
            e5[0], e5[4] = ce[i][0], ce[i][1]
            call(e5)
        torch.cuda.synchronize()
        cms = float(np.median([elapsed_ms(L, a, b) for a, b in ce]))
        for a, b in ce:
            L.hipEventDestroy(a)
            L.hipEventDestroy(b)
        del flush
        cold = {"ms_per_call_median": cms, "tokens_per_s": T / (cms / 1e3),
                "flush_read_bytes": 512 << 20, "calls": cold_calls}

    return dict(wl=wl, ms_total=ms_total, K=K, wall=wall, phase_ms=phase_ms, dom=dom,
                dom_ms=dom_ms, cold=cold, form=form)


def state_form(wl, cp):
    """The state pass's operand form for this call, as the library chooses it
    (for the implementation byte model only): context parallelism (cp, seen
    from the workspace size), else the T form for 16-bit D = 128 calls with
    more column tiles than CUs or W-form intermediates past 200 MiB."""
    import torch
    from gated_deltanet_chunked_varlen_amd import _native as nat
    if cp:
        return "context parallel (W form)"
    if wl.dtype == "f32" or wl.D != 128:
        return "W form"
    H, D = wl.H, wl.D
    hq, hk = wl.q.shape[1], wl.k.shape[1]
    cap = int(nat.lib().gdn_max_chunks(wl.T, wl.N))
    inter = cap * (H * (2 * 64 * D + 64 * 64) + (hk + hq) * 64 * D) * 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return "T form" if (wl.N * H * (D // 16) > cus or inter > (200 << 20)) else "W form"


def prefill_record(m):
    """The figures of one measured prefill workload (measure_prefill)."""
    wl = m["wl"]
    H, D, N, T = wl.H, wl.D, wl.N, wl.T
    K, ms_total, phase_ms, dom, dom_ms = m["K"], m["ms_total"], m["phase_ms"], m["dom"], m["dom_ms"]
    ms_step = ms_total / K
    tokens_per_s = T * K / (ms_total / 1e3)
    # the whole call: counter-measured HBM bytes of every kernel it launches
    # (where the committed counters match the kernel sources) over the
    # measured time per step
    per_phase = {ph: load_traffic(ph, wl.name) for ph in PHASES if phase_ms[ph] > 0.0}
    known = {ph: b for ph, b in per_phase.items() if b is not None}
    call_traffic = None
    if known and set(known) >= {"intra", "state"}:
        tb = sum(known.values())
        gbs = tb / (ms_step / 1e3) / 1e9
        call_traffic = {"bytes": tb, "phases": sorted(known), "achieved": gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "source": TRAFFIC_SOURCE}
    flops = T * H * FLOPS_PER_TOKEN_HEAD(D)
    tflops = flops / (ms_step / 1e3) / 1e12
    peak_mm = FP32_PEAK_TFLOPS if wl.dtype == "f32" else BF16_PEAK_TFLOPS   # fp16 peak = bf16 peak
    mbytes = method_bytes(wl)
    achieved = mbytes / (dom_ms / 1e3) / 1e9
    impl_bytes = per_token_head_bytes(wl, dom, m["form"] == "T form") * T * H
    traffic = load_traffic(dom, wl.name)
    return {
        "ms_per_step": ms_step,
        "tokens_per_s": tokens_per_s,
        "tflops_canonical": tflops,
        "tflops_triangle": T * H * FLOPS_TRI_PER_TOKEN_HEAD(D) / (ms_step / 1e3) / 1e12,
        "mfma_peak_frac": tflops / peak_mm,
        "phase_ms_warmup": phase_ms,
        "mfma_counters": load_mfma(wl.name) or None,
        "state_pass_form": m["form"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_source": TRAFFIC_SOURCE if traffic else None,
                     "avg_launch_ms": dom_ms,
                     "timing": "HIP events around the kernel in each of K further steps",
                     "algorithmic_bytes_per_launch": mbytes,
                     "algorithmic_bytes_model": "method bytes of the whole call (q, k, v, o, "
                                                "g, beta, states, checkpoints) over the "
                                                "dominant kernel's time",
                     "implementation_bytes_per_launch": impl_bytes,
                     "implementation_frac": impl_bytes / (dom_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "call_hbm_frac_method_bytes": mbytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "cold_cache": m["cold"],
        "call_traffic": call_traffic,
        "wall_s_timed": m["wall"],
    }


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        summarize(sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        summarize_mfma(sys.argv[2:])
        return
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="gva8 (default, the headline; also times varlen2x2048 "
                         "under \"varlen_2x2048\"); varlen2x2048, single128, "
                         "ragged6, long262144 alone; decode for the decode step "
                         "(its own JSON line)")
    ap.add_argument("--no-extra", action="store_true",
                    help="with the default workload, skip the 2 x 2048 figures")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="calls timed after flushing the last-level cache (0: none)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: the library runs on one GPU only (more GPUs would "
                  "take whole sequences or heads each, with no communication); "
                  "--gpus %d is not supported" % args.gpus,
                  file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "decode":
        bench_decode(args)
        return

    from gated_deltanet_chunked_varlen_amd import workloads as W
    wl = W.WORKLOADS[args.workload]()
    m = measure_prefill(wl, args.steps, args.warmup, args.cold_calls)
    r = prefill_record(m)
    H, D, N, T = wl.H, wl.D, wl.N, wl.T
    res = {
        "metric": "GDN prefill tokens/s (all heads) + % of MI355X bf16 MFMA peak, H=16 D=128",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded numpy draws, see workloads.py)",
        "config": {"workload": wl.name, "num_seqs": N, "seq_lens": wl.lengths,
                   "total_tokens": T, "num_q_heads": int(wl.q.shape[1]),
                   "num_k_heads": int(wl.k.shape[1]), "num_v_heads": int(wl.v.shape[1]),
                   "head_size": D, "qk_l2norm_in_kernel": wl.l2norm_in_kernel,
                   "checkpoint_every_n_tokens": wl.checkpoint_every,
                   "parallelism": "single GPU"},
    }
    res.update({k: v for k, v in r.items() if k not in ("ms_per_step", "tokens_per_s")})
    if args.workload == DEFAULT_WORKLOAD and not args.no_extra:
        # context parallelism: one 65 536-token sequence with 4 heads, the
        # ordinary pass against the context-parallel one ("auto" takes it)
        wc = W.WORKLOADS["long65536h4"]()
        k_cp = max(1, min(args.steps, 50))
        m_off = measure_prefill(wc, k_cp, min(args.warmup, 50), 0, use_cp=False)
        m_cp = measure_prefill(wc, k_cp, min(args.warmup, 50), 0, use_cp="auto")
        ms_off, ms_cp = m_off["ms_total"] / m_off["K"], m_cp["ms_total"] / m_cp["K"]
        res["context_parallel_1x65536_h4"] = {
            "workload": wc.name, "steps": k_cp,
            "ms_per_step_cp": ms_cp, "ms_per_step_no_cp": ms_off,
            "speedup": ms_off / ms_cp,
            "tokens_per_s_cp": wc.T / (ms_cp * 1e-3),
            "phase_ms_warmup_cp": m_cp["phase_ms"],
            "note": "the state phase holds the segment transitions, the start-state "
                    "fix-up and the fused pass over all segments"}

        # the 2 x 2048-token, 16-head batch, timed the same way in this run
        w2 = W.WORKLOADS["varlen2x2048"]()
        r2 = prefill_record(measure_prefill(w2, args.steps, min(args.warmup, 500), 0))
        res["varlen_2x2048"] = {
            "workload": w2.name, "ms_per_step": r2["ms_per_step"],
            "tokens_per_s": r2["tokens_per_s"], "tflops_canonical": r2["tflops_canonical"],
            "mfma_peak_frac": r2["mfma_peak_frac"], "phase_ms_warmup": r2["phase_ms_warmup"],
            "roofline": r2["roofline"],
            "call_hbm_frac_method_bytes": r2["call_hbm_frac_method_bytes"]}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
