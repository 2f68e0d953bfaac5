"""Seeded synthetic inputs for the GDN prefill workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the method's arithmetic.  Both the HIP path's tests/bench and
the CPU oracle take their inputs from here.

Draws per workload: ``numpy.random.SeedSequence(seed)`` spawns one child per
draw, in this order: lengths, q, k, v, alpha, beta, initial state, pool slot
permutation.  Each child drives a PCG64 generator; normal arrays are drawn in
blocks of 2**22 values, block b from the b-th grandchild of its child (so the
values do not depend on how many threads draw them).  Values are drawn in
fp32; bf16 workloads round them once (round to nearest even) and both sides
use the rounded values.  "L2-normalised in the generator" divides each token's
fp32 vector by its Euclidean norm before the rounding; that is part of the
input recipe, not the kernel's in-kernel normalisation.

The shapes follow the pages' examples: gitcode "FlashInfer GDN Prefill
完全指南" (section "基础用法": 2 x 2048 tokens, 16 heads, head size 128;
section "状态池": a 64-slot fp32 pool; section "中间状态检查点": checkpoints
every n tokens) and weigao.cc "GDN 与 Chunked Prefill" (section "chunked
prefill 有两层含义": sequences of 130, 20 and 300 tokens).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


def _round_bf16_inplace(x: np.ndarray) -> np.ndarray:
    """Round a C-contiguous fp32 array to the nearest-even bf16 value in
    place (finite values), block by block on threads."""
    from concurrent.futures import ThreadPoolExecutor
    flat = x.reshape(-1).view(np.uint32)
    step = 1 << 22

    def work(s):
        b = flat[s:s + step]
        lsb = (b >> 16) & 1
        b += 0x7FFF
        b += lsb
        b &= 0xFFFF0000

    starts = range(0, flat.size, step)
    if len(starts) > 1:
        with ThreadPoolExecutor(16) as ex:
            list(ex.map(work, starts))
    else:
        for s in starts:
            work(s)
    return x


def round_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even IEEE half, returned as fp32 holding the fp16
    values (numpy's conversion rounds to nearest even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_fp8(x: np.ndarray, fmt: str) -> np.ndarray:
    """fp32 values rounded to the 8-bit float format ``fmt`` ("e4m3": OCP
    E4M3, "e5m2") by torch's CPU conversion (nearest, ties to even), returned
    as fp32.  Used for fp8 state inputs only; values here are far inside the
    formats' ranges."""
    import torch
    dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dt).to(torch.float32).numpy()


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as a new fp32 array holding the
    bf16 values (finite inputs)."""
    return _round_bf16_inplace(np.array(x, dtype=np.float32, copy=True, order="C"))


_BLOCK = 1 << 22


def _normal(seq: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) array, drawn block by block (threads in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    nb = (flat.size + _BLOCK - 1) // _BLOCK
    kids = seq.spawn(nb)

    def work(b):
        g = np.random.Generator(np.random.PCG64(kids[b]))
        blk = flat[b * _BLOCK:(b + 1) * _BLOCK]
        g.standard_normal(out=blk, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)

    if nb > 1:
        with ThreadPoolExecutor(min(16, nb)) as ex:
            list(ex.map(work, range(nb)))
    elif nb == 1:
        work(0)
    return out


def _gen(seq: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seq))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """Divide each vector (last axis) by its Euclidean norm, block by block."""
    out = np.empty_like(x, dtype=np.float32)
    step = max(1, (1 << 22) // max(1, x.shape[-1] * x.shape[-2]))
    for s in range(0, x.shape[0], step):
        blk = x[s:s + step].astype(np.float64)
        n = np.sqrt(np.sum(blk * blk, axis=-1, keepdims=True))
        out[s:s + step] = (blk / n).astype(np.float32)
    return out


@dataclass
class Workload:
    """One call's inputs.  Arrays are fp32 holding values exactly
    representable in ``dtype`` (``"bf16"``, ``"f16"`` or ``"f32"``)."""
    name: str
    dtype: str
    cu_seqlens: np.ndarray                  # [N+1] int32 or int64
    q: np.ndarray                           # [T, hq, D]
    k: np.ndarray                           # [T, hk, D]
    v: np.ndarray                           # [T, hv, D]
    g: Optional[np.ndarray]                 # [T, H] fp32 (alpha)
    beta: Optional[np.ndarray]              # [T, H] fp32
    scale: Optional[float] = None
    l2norm_in_kernel: bool = False
    initial_state: Optional[np.ndarray] = None   # [rows, H, D, D]
    initial_state_dtype: str = "f32"
    state_indices: Optional[np.ndarray] = None   # [N]
    output_final_state: bool = True
    final_state_dtype: str = "f32"
    in_place_pool: bool = False
    checkpoint_every: int = 0
    checkpoint_cu_starts: Optional[np.ndarray] = None
    checkpoint_dtype: str = "f32"
    notes: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def N(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def H(self) -> int:
        return max(int(self.q.shape[1]), int(self.v.shape[1]))

    @property
    def D(self) -> int:
        return int(self.q.shape[2])

    @property
    def lengths(self) -> List[int]:
        cu = self.cu_seqlens
        return [int(cu[i + 1] - cu[i]) for i in range(self.N)]


def _cu(lengths, dtype=np.int32):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(dtype)


def make(seed: int, lengths, hq: int, hk: int, hv: int, D: int,
         dtype: str = "bf16", *, alpha_range=(0.9, 1.0), gates: bool = True,
         normalise_in_generator: bool = False, l2norm_in_kernel: bool = False,
         scale: Optional[float] = None, init: Optional[str] = None,
         init_std: float = 0.02, init_dtype: str = "f32",
         pool_size: Optional[int] = None, in_place_pool: bool = False,
         checkpoint_every: int = 0, final_state_dtype: str = "f32",
         checkpoint_dtype: str = "f32",
         cu_dtype=np.int32, name: str = "custom", qkv_std: float = 1.0,
         draw_lengths=None) -> Workload:
    """General seeded workload.  ``init`` is None (zero state), "seq" (one
    state per sequence) or "pool" (a pool of ``pool_size`` rows addressed by
    a random unique ``state_indices``)."""
    kids = np.random.SeedSequence(seed).spawn(8)
    if draw_lengths is not None:
        lengths = draw_lengths(_gen(kids[0]))
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    H = max(hq, hv)
    q = _normal(kids[1], (T, hq, D), qkv_std)
    k = _normal(kids[2], (T, hk, D), qkv_std)
    v = _normal(kids[3], (T, hv, D), qkv_std)
    if normalise_in_generator:
        q, k = _unit_rows(q), _unit_rows(k)
    if gates:
        lo, hi = alpha_range
        g = _gen(kids[4]).uniform(lo, hi, size=(T, H)).astype(np.float32)
        x = _gen(kids[5]).standard_normal(size=(T, H)).astype(np.float32)
        beta = (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)
    else:
        g = beta = None
    init_state = sidx = None
    if init == "seq":
        init_state = _normal(kids[6], (len(lengths), H, D, D), init_std)
    elif init == "pool":
        assert pool_size is not None and pool_size >= len(lengths)
        init_state = _normal(kids[6], (pool_size, H, D, D), init_std)
        sidx = _gen(kids[7]).permutation(pool_size)[:len(lengths)].astype(np.int32)
    if init_state is not None and init_dtype == "bf16":
        init_state = _round_bf16_inplace(init_state)
    if init_state is not None and init_dtype == "f16":
        init_state = round_f16(init_state)
    if init_state is not None and init_dtype in ("e4m3", "e5m2"):
        init_state = round_fp8(init_state, init_dtype)
    if dtype == "bf16":
        q, k, v = (_round_bf16_inplace(q), _round_bf16_inplace(k),
                   _round_bf16_inplace(v))
    elif dtype == "f16":
        q, k, v = round_f16(q), round_f16(k), round_f16(v)
    cu = _cu(lengths, cu_dtype)
    ccs = None
    if checkpoint_every > 0:
        ccs = _cu([L // checkpoint_every for L in lengths], cu_dtype)
    return Workload(name=name, dtype=dtype, cu_seqlens=cu, q=q, k=k, v=v,
                    g=g, beta=beta, scale=scale,
                    l2norm_in_kernel=l2norm_in_kernel,
                    initial_state=init_state, initial_state_dtype=init_dtype,
                    state_indices=sidx, final_state_dtype=final_state_dtype,
                    in_place_pool=in_place_pool,
                    checkpoint_every=checkpoint_every,
                    checkpoint_cu_starts=ccs, checkpoint_dtype=checkpoint_dtype)



# ---------------------------------------------------------------- to device

def state_torch_dtype(name):
    """torch dtype of a state dtype name."""
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
            "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[name]


def to_device(wl, device="cuda"):
    """The workload's inputs as device tensors in their storage dtypes (a
    copy, nothing computed): q, k, v, g, beta, cu_seqlens, initial_state,
    state_indices and checkpoint_cu_starts (None where the workload has
    none)."""
    import torch
    qdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[wl.dtype]

    def t(a, dt):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

    def idx(a):
        return None if a is None else torch.from_numpy(a.copy()).to(device)

    return dict(
        q=t(wl.q, qdt), k=t(wl.k, qdt), v=t(wl.v, qdt),
        g=t(wl.g, torch.float32), beta=t(wl.beta, torch.float32),
        cu_seqlens=idx(wl.cu_seqlens),
        initial_state=t(wl.initial_state, state_torch_dtype(wl.initial_state_dtype)),
        state_indices=idx(wl.state_indices),
        checkpoint_cu_starts=idx(wl.checkpoint_cu_starts),
    )


# The five named workloads, seeds 1000 + index.

def single_l128_h1_d32_f32() -> Workload:
    """1 sequence of 128 tokens (2 chunks), 1 head, head size 32, fp32,
    q/k unit rows from the generator, alpha ~ U[0.9, 1], beta = sigmoid(N(0,1)),
    scale 1/sqrt(32), zero initial state."""
    return make(1000, [128], 1, 1, 1, 32, "f32", normalise_in_generator=True,
                scale=1.0 / np.sqrt(32.0), name="single_L128_h1_d32_f32")


def varlen_2x2048_h16_d128() -> Workload:
    """2 x 2048 tokens, 16 heads, head size 128, bf16, in-kernel q/k L2
    norm, alpha ~ U[0.9, 1], zero initial state, fp32 final state."""
    return make(1001, [2048, 2048], 16, 16, 16, 128, "bf16",
                l2norm_in_kernel=True, name="varlen_2x2048_h16_d128_bf16")


def ragged6_pool64_h16_d128() -> Workload:
    """Lengths [130, 20, 300, 0, 64, 1], 16 heads, head size 128, bf16,
    in-kernel q/k L2 norm, fp32 64-slot pool ~ N(0, 0.02) read and written in
    place through unique state_indices."""
    return make(1002, [130, 20, 300, 0, 64, 1], 16, 16, 16, 128, "bf16",
                l2norm_in_kernel=True, init="pool", pool_size=64,
                in_place_pool=True, name="ragged6_pool64_h16_d128_bf16")


def gva8_h16x32_d128_checkpoints() -> Workload:
    """8 sequences with lengths ~ U[1, 8192], 16 q/k heads and 32 v heads,
    head size 128, bf16, alpha ~ U[0.85, 1], in-kernel q/k L2 norm,
    checkpoints every 1024 tokens, fp32 final states."""
    return make(1003, None, 16, 16, 32, 128, "bf16", alpha_range=(0.85, 1.0),
                l2norm_in_kernel=True, checkpoint_every=1024,
                draw_lengths=lambda rng: rng.integers(1, 8193, size=8),
                name="gva8_h16x32_d128_bf16_ckpt1024")


def long_l262144_h32_d128() -> Workload:
    """One sequence of 262144 tokens (4096 chunks), 32 heads, head size 128,
    bf16, q/k unit rows from the generator, alpha ~ U[0.95, 1], bf16 initial
    state ~ N(0, 0.02), fp32 final state."""
    return make(1004, [262144], 32, 32, 32, 128, "bf16",
                alpha_range=(0.95, 1.0), normalise_in_generator=True,
                init="seq", init_dtype="bf16",
                name="long_L262144_h32_d128_bf16")


def long_l65536_h4_d128() -> Workload:
    """One sequence of 65536 tokens (1024 chunks) with 4 heads, head size 128,
    bf16, in-kernel q/k L2 norm, alpha ~ U[0.9, 1], fp32 initial and final
    states: a long prompt with too few (sequence, head) pairs to fill the GPU,
    the shape context parallelism is for."""
    return make(1006, [65536], 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                init="seq", init_std=0.02, name="long_L65536_h4_d128_bf16")


def decode_batch() -> Workload:
    """One decode step for 256 sequences (one new token each), 16 heads, head
    size 128, bf16, in-kernel q/k L2 norm, alpha ~ U[0.9, 1], fp32 512-slot
    state pool ~ N(0, 0.02) read and written in place through unique
    state_indices (the serving shape of the prefill's pool)."""
    return make(1005, [1] * 256, 16, 16, 16, 128, "bf16",
                l2norm_in_kernel=True, init="pool", pool_size=512,
                in_place_pool=True, name="decode_b256_h16_d128_bf16_pool512")


WORKLOADS = {
    "single128": single_l128_h1_d32_f32,
    "varlen2x2048": varlen_2x2048_h16_d128,
    "ragged6": ragged6_pool64_h16_d128,
    "gva8": gva8_h16x32_d128_checkpoints,
    "long262144": long_l262144_h32_d128,
    "long65536h4": long_l65536_h4_d128,
    "decode": decode_batch,
}
