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


def block_max_rel_l2(x, ref, blocks):
    """Largest relative L2 error over the given blocks: ``blocks`` is a list
    of index expressions into the leading axes of x / ref.  A block's error
    is ||x_b - ref_b|| over the larger of ||ref_b|| and the norm the block
    would have at the whole tensor's root-mean-square value.  The floor is
    what the rounding of the inputs allows: a dot product of rounded operands
    errs in proportion to the sum of the magnitudes of its terms, not to its
    value, so a block whose true values nearly cancel (a one-token output
    whose q and k are nearly orthogonal) is held to the tensor's scale.  A
    block that is wrong at the tensor's scale (zeroed, swapped, misplaced)
    still reads close to 1.  Returns (error, the block where it occurs)."""
    ref = np.asarray(ref, np.float64)
    x = np.asarray(x, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    worst, where = 0.0, None
    for b in blocks:
        rb, xb = ref[b], x[b]
        den = max(float(np.linalg.norm(rb)), rms * np.sqrt(rb.size))
        e = float(np.linalg.norm(xb - rb)) / den if den > 0 else float(np.linalg.norm(xb))
        if e > worst:
            worst, where = e, b
    return worst, where


def chunk_blocks(cu, H, C=64):
    """(token slice, head) of every C-token chunk of every sequence (chunks
    start at each sequence's first token) and every head."""
    cu = np.asarray(cu, np.int64)
    out = []
    for i in range(len(cu) - 1):
        for t0 in range(int(cu[i]), int(cu[i + 1]), C):
            t1 = min(t0 + C, int(cu[i + 1]))
            out.extend((slice(t0, t1), h) for h in range(H))
    return out


def sequence_blocks(cu):
    cu = np.asarray(cu, np.int64)
    return [slice(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)
            if cu[i + 1] > cu[i]]


def compare(wl, gpu, orc, heads=None):
    """Relative L2 errors of outputs / final states / checkpoints, each over
    the whole tensor and, as "<name>_block", the largest over every
    (64-token chunk, head) block and every sequence of the output, every
    (sequence, head) of the final state and every (row, head) of the
    checkpoints: a wrong chunk, head or row cannot hide in a large tensor."""
    tol = TOL[wl.dtype]
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    go = sel(gpu["out"])
    ro = orc["out"]
    nh = ro.shape[1]
    errs = {"out": rel_l2(go, ro)}
    e1, _ = block_max_rel_l2(go, ro, chunk_blocks(wl.cu_seqlens, nh))
    e2, _ = block_max_rel_l2(go, ro, sequence_blocks(wl.cu_seqlens))
    errs["out_block"] = max(e1, e2)
    if wl.output_final_state:
        if wl.state_indices is not None:
            idx = [int(r) for r in wl.state_indices]
            gf = sel(gpu["final"][idx])
        else:
            gf = sel(gpu["final"])
        rf = orc["final"]
        errs["final"] = rel_l2(gf, rf)
        nz = [(i, h) for i in range(rf.shape[0]) for h in range(nh)
              if np.any(rf[i, h] != 0)]
        errs["final_block"] = block_max_rel_l2(gf, rf, nz)[0] if nz else 0.0
    if wl.checkpoint_every > 0 and orc["ckpt"] is not None and orc["ckpt"].size:
        gc, rc = sel(gpu["ckpt"]), orc["ckpt"]
        errs["ckpt"] = rel_l2(gc, rc)
        errs["ckpt_block"] = block_max_rel_l2(
            gc, rc, [(r, h) for r in range(rc.shape[0]) for h in range(nh)])[0]
    return errs, tol


def bars(wl):
    """The relative-L2 bar of each compared tensor: the compute bar, plus the
    store rounding for states kept in a type narrower than fp32.  The block
    maxima (``*_block``) take the same bars."""
    tol = TOL[wl.dtype]
    b = {"out": tol,
         "final": tol + STORE_TOL.get(wl.final_state_dtype, 0.0),
         "ckpt": tol + STORE_TOL.get(wl.checkpoint_dtype, 0.0)}
    b.update({k + "_block": v for k, v in list(b.items())})
    return b
