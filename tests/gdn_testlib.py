"""Shared helpers for the tests: run a workload through the HIP path (via the
C ABI binding) and through the CPU oracle, and compare.

Tolerances (relative L2 over each whole tensor, fp64): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs with fp32 accumulation, and for fp16 inputs the bf16 bar
scaled by the ratio of the two formats' unit roundoffs (2^-11 / 2^-8): the
error comes from rounding the stored 16-bit intermediates, which scales with
the unit roundoff.
"""
from __future__ import annotations

import numpy as np

from gated_deltanet_chunked_varlen_amd import workloads as W
from oracle import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2 / 8}

# A state stored in a narrower type than fp32 carries, on top of the bar of
# its computation, the rounding of every element to that type: at most the
# type's unit roundoff relative to the element (2^-8 bf16, 2^-11 fp16, 2^-4
# E4M3 with 3 mantissa bits, 2^-3 E5M2 with 2), so at most that in relative
# L2.
STORE_TOL = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11,
             "e4m3": 2.0 ** -4, "e5m2": 2.0 ** -3}

state_torch_dtype = W.state_torch_dtype


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm((x - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    return float(d / n) if n > 0 else float(d)


def oracle_problem(wl, heads=None):
    """The oracle's view of a workload.  With ``heads``, only those sab heads
    are kept: each keeps its own copy of the q/k/v head it reads (an exact
    copy of the inputs; no arithmetic), so the oracle sees a smaller problem
    whose head j is sab head heads[j]."""
    q, k, v, g, beta, init = wl.q, wl.k, wl.v, wl.g, wl.beta, wl.initial_state
    if heads is not None:
        H = wl.H
        src = lambda x: [h // (H // x.shape[1]) for h in heads]
        q, k, v = q[:, src(q)], k[:, src(k)], v[:, src(v)]
        g = None if g is None else g[:, heads]
        beta = None if beta is None else beta[:, heads]
        init = None if init is None else init[:, heads]
    return oracle.Problem(
        q=q, k=k, v=v, cu=wl.cu_seqlens.astype(np.int64), g=g,
        beta=beta, scale=wl.scale, l2norm=wl.l2norm_in_kernel,
        init_state=init,
        state_indices=None if wl.state_indices is None else wl.state_indices.astype(np.int64),
        ckpt_every=wl.checkpoint_every,
        ckpt_cu_starts=None if wl.checkpoint_cu_starts is None
        else wl.checkpoint_cu_starts.astype(np.int64))


def run_oracle(wl, heads=None):
    """Oracle outputs; with ``heads`` the head axis holds only those heads."""
    return oracle.token(oracle_problem(wl, heads))


# ------------------------------------------------------------------ GPU side

def _torch():
    import torch
    return torch


to_device = W.to_device


def run_gpu(wl, device="cuda", status=False, **over):
    """Run the HIP path; returns numpy fp64 arrays (out, final, ckpt, pool)."""
    torch = _torch()
    from gated_deltanet_chunked_varlen_amd import chunk_gated_delta_rule
    d = to_device(wl, device)
    H, D, N = wl.H, wl.D, wl.N
    kw = dict(g=d["g"], beta=d["beta"], scale=wl.scale,
              cu_seqlens=d["cu_seqlens"],
              use_qk_l2norm_in_kernel=wl.l2norm_in_kernel,
              output_final_state=wl.output_final_state)
    pool_before = None
    if wl.state_indices is not None:
        pool = d["initial_state"]
        pool_before = pool.clone()
        kw.update(initial_state=pool, state_indices=d["state_indices"],
                  output_state=pool if wl.in_place_pool else torch.zeros_like(pool))
    else:
        kw.update(initial_state=d["initial_state"])
        if wl.output_final_state:
            kw.update(output_state=torch.zeros((N, H, D, D), dtype=torch.float32, device=device)
                      .to(state_torch_dtype(wl.final_state_dtype)))
    ck = None
    if wl.checkpoint_every > 0:
        rows = int(wl.checkpoint_cu_starts[-1])
        ck = torch.zeros((rows, H, D, D), dtype=torch.float32, device=device).to(
            state_torch_dtype(wl.checkpoint_dtype))
        kw.update(state_checkpoints=ck, checkpoint_cu_starts=d["checkpoint_cu_starts"],
                  checkpoint_every_n_tokens=wl.checkpoint_every)
    st = torch.full((1,), -1, dtype=torch.int32, device=device) if status else None
    if st is not None:
        kw["status"] = st
    kw.update(over)
    res = chunk_gated_delta_rule(d["q"], d["k"], d["v"], **kw)
    out, fin = (res if wl.output_final_state else (res, None))
    torch.cuda.synchronize()
    f64 = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)
    r = dict(out=f64(out), final=f64(fin), ckpt=f64(ck),
             pool_before=f64(pool_before))
    if st is not None:
        r["status"] = int(st.item())
    return r


def expected_pool(wl, orc_final):
    """The pool after the call: rows state_indices[i] replaced by sequence
    i's final state, every other row unchanged."""
    pool = wl.initial_state.astype(np.float64).copy()
    for i, r in enumerate(wl.state_indices):
        pool[int(r)] = orc_final[i]
    return pool


def run_gpu_decode(wl, device="cuda", status=False, **over):
    """One decode step on the HIP path for a workload whose sequences all have
    length 1 (token i = sequence i); same return dict as run_gpu.  Keyword
    overrides replace the call's arguments (e.g. strided state views)."""
    torch = _torch()
    from gated_deltanet_chunked_varlen_amd import gated_delta_rule_decode
    assert all(int(x) == 1 for x in np.diff(wl.cu_seqlens))
    d = to_device(wl, device)
    H, D, N = wl.H, wl.D, wl.N
    kw = dict(g=d["g"], beta=d["beta"], scale=wl.scale,
              use_qk_l2norm_in_kernel=wl.l2norm_in_kernel,
              output_final_state=wl.output_final_state)
    pool_before = None
    if wl.state_indices is not None:
        pool = d["initial_state"]
        pool_before = pool.clone()
        kw.update(initial_state=pool, state_indices=d["state_indices"],
                  output_state=pool if wl.in_place_pool else torch.zeros_like(pool))
    else:
        kw.update(initial_state=d["initial_state"])
        if wl.output_final_state:
            kw.update(output_state=torch.zeros((N, H, D, D), dtype=torch.float32, device=device)
                      .to(state_torch_dtype(wl.final_state_dtype)))
    st = torch.full((1,), -1, dtype=torch.int32, device=device) if status else None
    if st is not None:
        kw["status"] = st
    kw.update(over)
    res = gated_delta_rule_decode(d["q"], d["k"], d["v"], **kw)
    out, fin = (res if wl.output_final_state else (res, None))
    torch.cuda.synchronize()
    f64 = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)
    r = dict(out=f64(out), final=f64(fin), ckpt=None, pool_before=f64(pool_before))
    if st is not None:
        r["status"] = int(st.item())
    return r


def compare(wl, gpu, orc, heads=None):
    """Relative L2 errors of outputs / final states / checkpoints."""
    tol = TOL[wl.dtype]
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    errs = {"out": rel_l2(sel(gpu["out"]), orc["out"])}
    if wl.output_final_state:
        if wl.state_indices is not None:
            idx = [int(r) for r in wl.state_indices]
            errs["final"] = rel_l2(sel(gpu["final"][idx]), orc["final"])
        else:
            errs["final"] = rel_l2(sel(gpu["final"]), orc["final"])
    if wl.checkpoint_every > 0 and orc["ckpt"] is not None and orc["ckpt"].size:
        errs["ckpt"] = rel_l2(sel(gpu["ckpt"]), orc["ckpt"])
    return errs, tol


def bars(wl):
    """The relative-L2 bar of each compared tensor: the compute bar, plus the
    store rounding for states kept in a type narrower than fp32."""
    tol = TOL[wl.dtype]
    return {"out": tol,
            "final": tol + STORE_TOL.get(wl.final_state_dtype, 0.0),
            "ckpt": tol + STORE_TOL.get(wl.checkpoint_dtype, 0.0)}
