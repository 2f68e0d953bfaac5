"""Seeded synthetic inputs for the GDN prefill workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the method's arithmetic.  Both the HIP path's tests/bench and
the CPU oracle take their inputs from here.

Draw order per workload, from ``numpy.random.default_rng(seed)``: lengths,
q, k, v, alpha, beta, initial state, pool slot permutation.  Values are drawn
in fp32; bf16 workloads round them once (round to nearest even) and both sides
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


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as fp32 holding the bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def _normal(rng, shape, dtype=np.float32):
    return rng.standard_normal(size=shape, dtype=np.float32).astype(dtype)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


@dataclass
class Workload:
    """One call's inputs.  Arrays are fp32 holding values exactly
    representable in ``dtype`` (``"bf16"`` or ``"f32"``)."""
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
         cu_dtype=np.int32, name: str = "custom", qkv_std: float = 1.0,
         draw_lengths=None) -> Workload:
    """General seeded workload.  ``init`` is None (zero state), "seq" (one
    state per sequence) or "pool" (a pool of ``pool_size`` rows addressed by
    a random unique ``state_indices``)."""
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lengths = draw_lengths(rng)
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    H = max(hq, hv)
    q = _normal(rng, (T, hq, D)) * qkv_std
    k = _normal(rng, (T, hk, D)) * qkv_std
    v = _normal(rng, (T, hv, D)) * qkv_std
    if normalise_in_generator:
        q, k = _unit_rows(q), _unit_rows(k)
    if gates:
        lo, hi = alpha_range
        g = rng.uniform(lo, hi, size=(T, H)).astype(np.float32)
        x = rng.standard_normal(size=(T, H)).astype(np.float32)
        beta = (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)
    else:
        g = beta = None
    init_state = sidx = None
    if init == "seq":
        init_state = (rng.standard_normal(size=(len(lengths), H, D, D),
                                          dtype=np.float32) * init_std)
    elif init == "pool":
        assert pool_size is not None and pool_size >= len(lengths)
        init_state = (rng.standard_normal(size=(pool_size, H, D, D),
                                          dtype=np.float32) * init_std)
        sidx = rng.permutation(pool_size)[:len(lengths)].astype(np.int32)
    if init_state is not None and init_dtype == "bf16":
        init_state = round_bf16(init_state)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
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
                    checkpoint_cu_starts=ccs)


# The five named workloads, seeds 1000 + index.

def c1_single_small() -> Workload:
    """1 sequence of 128 tokens (2 chunks), 1 head, head size 32, fp32,
    q/k unit rows from the generator, alpha ~ U[0.9, 1], beta = sigmoid(N(0,1)),
    scale 1/sqrt(32), zero initial state."""
    return make(1000, [128], 1, 1, 1, 32, "f32", normalise_in_generator=True,
                scale=1.0 / np.sqrt(32.0), name="single_L128_h1_d32_f32")


def c2_two_by_2048() -> Workload:
    """2 x 2048 tokens, 16 heads, head size 128, bf16, in-kernel q/k L2
    norm, alpha ~ U[0.9, 1], zero initial state, fp32 final state."""
    return make(1001, [2048, 2048], 16, 16, 16, 128, "bf16",
                l2norm_in_kernel=True, name="varlen_2x2048_h16_d128_bf16")


def c3_ragged_pool() -> Workload:
    """Lengths [130, 20, 300, 0, 64, 1], 16 heads, head size 128, bf16,
    in-kernel q/k L2 norm, fp32 64-slot pool ~ N(0, 0.02) read and written in
    place through unique state_indices."""
    return make(1002, [130, 20, 300, 0, 64, 1], 16, 16, 16, 128, "bf16",
                l2norm_in_kernel=True, init="pool", pool_size=64,
                in_place_pool=True, name="ragged6_pool64_h16_d128_bf16")


def c4_gva_checkpoints() -> Workload:
    """8 sequences with lengths ~ U[1, 8192], 16 q/k heads and 32 v heads,
    head size 128, bf16, alpha ~ U[0.85, 1], in-kernel q/k L2 norm,
    checkpoints every 1024 tokens, fp32 final states."""
    return make(1003, None, 16, 16, 32, 128, "bf16", alpha_range=(0.85, 1.0),
                l2norm_in_kernel=True, checkpoint_every=1024,
                draw_lengths=lambda rng: rng.integers(1, 8193, size=8),
                name="gva8_h16x32_d128_bf16_ckpt1024")


def c5_long_single() -> Workload:
    """One sequence of 262144 tokens (4096 chunks), 32 heads, head size 128,
    bf16, q/k unit rows from the generator, alpha ~ U[0.95, 1], bf16 initial
    state ~ N(0, 0.02), fp32 final state."""
    return make(1004, [262144], 32, 32, 32, 128, "bf16",
                alpha_range=(0.95, 1.0), normalise_in_generator=True,
                init="seq", init_dtype="bf16",
                name="long_L262144_h32_d128_bf16")


WORKLOADS = {
    "c1": c1_single_small,
    "c2": c2_two_by_2048,
    "c3": c3_ragged_pool,
    "c4": c4_gva_checkpoints,
    "c5": c5_long_single,
}
