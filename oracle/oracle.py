"""CPU oracle for the varlen chunked Gated Delta Rule prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` import this module.  It shares no code
with the HIP path (``gated_deltanet_chunked_varlen_amd``) and imports nothing
from it.

Three independent forms of the same definition live here:

* ``token`` / ``chunked`` -- ctypes front-ends of ``gdn_oracle.c`` (fp64 C).
  ``token`` is the recurrence itself (weigao.cc "GDN 与 Chunked Prefill",
  sections "GDN 是什么" and "块内 state 和块间 final state"; gitcode
  "FlashInfer GDN Prefill 完全指南", section "API 全参数解析"):
  ``S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T``,
  ``o_t = scale * S_t^T q_t``.  ``chunked`` is the chunk-wise rewrite with a
  unit-lower-triangular solve (weigao.cc, "递推公式如何展开成块内计算").
* ``exact_token`` -- the same recurrence in exact rational arithmetic
  (``fractions.Fraction``), for tiny sizes such as L = 8, D = 8, the first run
  0539edu "GDN与线性注意力GPU并行实现" section 3.1 recommends.
* ``chunk_factors`` -- one chunk's WY factors (A, T = (I + A)^-1, W, U) in
  numpy from the chunked form's definition, for checks of the GPU path's
  stored intermediates.
* ``partial_transition`` -- the pair-composition form of 0539edu sections
  2.1-2.2: each position is an affine pair ``(A_i, B_i)`` with
  ``A_i = a_i (I - b_i k_i k_i^T)``, ``B_i = b_i k_i v_i^T``; inside a chunk an
  inclusive scan of the pairs gives every position's map from the chunk's
  incoming state, and the chunk's composition carries the state on; outputs
  are scaled by ``scale``.

Parity is pinned for every function here by tests in ``tests/`` that check
against the pages' printed examples, closed forms and exact arithmetic.  The
head mapping, the L2-norm epsilon placement and the checkpoint row offset are
readings of the pages that no printed value fixes ("parity unpinned" by
value; they are tested for self-consistency only).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB names another build of gdn_oracle.c to load (e.g. one built with
# sanitizers); it is loaded as it is, never rebuilt
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")


def build(force: bool = True, out: str = _LIB, cc: str = "gcc", extra_flags=()) -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` (or ``out``) with gcc
    and OpenMP; ``cc`` and ``extra_flags`` serve instrumented builds."""
    if force or not os.path.exists(out) or (
            os.path.getmtime(out) < os.path.getmtime(_SRC)):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call([
            cc, "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
            "-Wall", "-Wextra", "-Wno-unused-parameter"] + list(extra_flags) + [
            _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("N", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hk", ctypes.c_int32),
        ("hv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("has_scale", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("cu", ctypes.c_void_p),
        ("l2norm", ctypes.c_int32),
        ("init_state", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p),
        ("state_rows", ctypes.c_int64),
        ("ckpt_every", ctypes.c_int64),
        ("ckpt_cu_starts", ctypes.c_void_p),
        ("heads", ctypes.c_void_p),
        ("n_heads", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or (
                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        L.oracle_chunk_table.restype = ctypes.c_int64
        L.oracle_chunk_table.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        L.oracle_checkpoint_starts.restype = None
        L.oracle_checkpoint_starts.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_gdn_token.restype = ctypes.c_int
        L.oracle_gdn_token.argtypes = [ctypes.POINTER(_Problem)] + [
            ctypes.c_void_p] * 3
        L.oracle_gdn_chunked.restype = ctypes.c_int
        L.oracle_gdn_chunked.argtypes = [
            ctypes.POINTER(_Problem), ctypes.c_int32] + [ctypes.c_void_p] * 5
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


@dataclass
class Problem:
    """One call's inputs, all as host arrays.

    q/k/v: [T, h, D] (any float dtype; converted exactly to fp64).
    g, beta: [T, H] or None.  cu: [N+1] integers.  init_state:
    [rows, H, D, D] in [v][k] element order, or None.  state_indices: [N] or
    None.  ckpt_every / ckpt_cu_starts as in the API.  heads: optional subset
    of sab heads to evaluate.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu: np.ndarray
    g: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    scale: Optional[float] = None
    l2norm: bool = False
    init_state: Optional[np.ndarray] = None
    state_indices: Optional[np.ndarray] = None
    ckpt_every: int = 0
    ckpt_cu_starts: Optional[np.ndarray] = None
    heads: Optional[Sequence[int]] = None
    _keep: list = field(default_factory=list, repr=False)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def N(self) -> int:
        return int(len(self.cu) - 1)

    @property
    def D(self) -> int:
        return int(self.q.shape[2])

    @property
    def H(self) -> int:
        return max(int(self.q.shape[1]), int(self.v.shape[1]))


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _i64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.int64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _struct(p: Problem):
    keep = []
    q, k, v = _f64(p.q), _f64(p.k), _f64(p.v)
    g, beta = _f64(p.g), _f64(p.beta)
    cu = _i64(p.cu)
    init = _f64(p.init_state)
    sidx = _i64(p.state_indices)
    ccs = _i64(p.ckpt_cu_starts)
    heads = None if p.heads is None else np.ascontiguousarray(
        p.heads, dtype=np.int32)
    keep += [q, k, v, g, beta, cu, init, sidx, ccs, heads]
    s = _Problem()
    s.T = q.shape[0]
    s.N = len(cu) - 1
    s.hq, s.hk, s.hv = q.shape[1], k.shape[1], v.shape[1]
    s.D = q.shape[2]
    s.q, s.k, s.v = _ptr(q), _ptr(k), _ptr(v)
    s.g, s.beta = _ptr(g), _ptr(beta)
    s.has_scale = 0 if p.scale is None else 1
    s.scale = 0.0 if p.scale is None else float(p.scale)
    s.cu = _ptr(cu)
    s.l2norm = 1 if p.l2norm else 0
    s.init_state = _ptr(init)
    s.state_indices = _ptr(sidx)
    s.state_rows = 0 if init is None else init.shape[0]
    s.ckpt_every = int(p.ckpt_every)
    s.ckpt_cu_starts = _ptr(ccs)
    s.heads = _ptr(heads)
    s.n_heads = 0 if heads is None else len(heads)
    return s, keep


def _outputs(p: Problem, want_ckpt: bool):
    T, H, D, N = p.T, p.H, p.D, p.N
    out = np.zeros((T, H, D), dtype=np.float64)
    final = np.zeros((N, H, D, D), dtype=np.float64)
    ck = None
    if want_ckpt and p.ckpt_every > 0:
        rows = int(checkpoint_starts(p.cu, p.ckpt_every)[-1])
        ck = np.zeros((rows, H, D, D), dtype=np.float64)
    return out, final, ck


def token(p: Problem) -> dict:
    """Token-by-token fp64 recurrence.  Returns out [T,H,D], final [N,H,D,D]
    (per sequence, [v][k]), ckpt [rows,H,D,D] or None."""
    s, keep = _struct(p)
    out, final, ck = _outputs(p, True)
    if p.ckpt_every > 0 and p.ckpt_cu_starts is None:
        raise ValueError("ckpt_cu_starts required")
    rc = lib().oracle_gdn_token(ctypes.byref(s), _ptr(out), _ptr(final),
                                _ptr(ck))
    if rc != 0:
        raise RuntimeError("oracle_gdn_token failed: %d" % rc)
    return {"out": out, "final": final, "ckpt": ck}


def chunked(p: Problem, C: int = 64, dump: bool = False) -> dict:
    """Chunked fp64 form with chunk size C; optionally the chunk-start states
    [n_chunks,H,D,D] and the new values nu [T,H,D]."""
    s, keep = _struct(p)
    out, final, ck = _outputs(p, True)
    cs = vn = None
    if dump:
        nch = int(chunk_table(p.cu, C)[2])
        cs = np.zeros((nch, p.H, p.D, p.D), dtype=np.float64)
        vn = np.zeros((p.T, p.H, p.D), dtype=np.float64)
    rc = lib().oracle_gdn_chunked(ctypes.byref(s), int(C), _ptr(out),
                                  _ptr(final), _ptr(ck), _ptr(cs), _ptr(vn))
    if rc != 0:
        raise RuntimeError("oracle_gdn_chunked failed: %d" % rc)
    return {"out": out, "final": final, "ckpt": ck, "chunk_states": cs,
            "vnew": vn}


def chunk_factors(p: Problem, h: int, t0: int, n: int) -> dict:
    """The WY factors of one chunk (tokens t0 .. t0 + n - 1 of one sequence)
    for sab head h, in fp64 (weigao.cc "GDN 与 Chunked Prefill", section
    "递推公式如何展开成块内计算"; 0539edu "GDN与线性注意力GPU并行实现",
    section 3.2).  With the gate log-cumsum inside the chunk
    G_t = sum_{s <= t} ln alpha_s, the keys k_t (L2-normalised when
    ``p.l2norm``, norm n_t; n_t = 1 otherwise) and beta_t:

        A[t, j] = beta_t exp(G_t - G_j) k_t . k_j   for j < t, else 0
        T       = (I + A)^-1
        W       = T diag(beta exp(G)) K,    U = T diag(beta) V

    and the chunk's new values are U - W S for S the state entering the chunk
    (as a D_k x D_v matrix).  Returns T, W, U, beta, G and the key norms n.
    Pinned against the C chunked form's new values (tests/test_oracle_pins.py)."""
    H = p.H
    kh = h // (H // p.k.shape[1])
    vh = h // (H // p.v.shape[1])
    K = np.asarray(p.k[t0:t0 + n, kh], np.float64)
    V = np.asarray(p.v[t0:t0 + n, vh], np.float64)
    if p.l2norm:
        nk = np.sqrt(np.sum(K * K, axis=1) + 1e-6)
        K = K / nk[:, None]
    else:
        nk = np.ones(n)
    alpha = np.ones(n) if p.g is None else np.asarray(p.g[t0:t0 + n, h], np.float64)
    beta = np.ones(n) if p.beta is None else np.asarray(p.beta[t0:t0 + n, h], np.float64)
    G = np.cumsum(np.log(alpha))
    A = np.tril(beta[:, None] * np.exp(G[:, None] - G[None, :]) * (K @ K.T), -1)
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ ((beta * np.exp(G))[:, None] * K)
    U = T @ (beta[:, None] * V)
    return {"T": T, "W": W, "U": U, "beta": beta, "G": G, "knorm": nk}


def chunk_table(cu, C: int = 64, cap: Optional[int] = None):
    """Flat chunk table (weigao.cc, "chunked prefill 有两层含义").

    Returns (table [n,2] int32 of (seq, chunk), cu_chunks [N+1] int32, n)."""
    cu = _i64(np.asarray(cu))
    N = len(cu) - 1
    if cap is None:
        cap = int(sum(max(0, (int(cu[i + 1] - cu[i]) + C - 1) // C)
                      for i in range(N)))
    table = np.zeros((max(cap, 1), 2), dtype=np.int32)
    cc = np.zeros(N + 1, dtype=np.int32)
    n = lib().oracle_chunk_table(_ptr(cu), N, int(C), _ptr(table), int(cap),
                                 _ptr(cc))
    if n < 0:
        raise ValueError("capacity too small")
    return table[:n], cc, int(n)


def checkpoint_starts(cu, every: int) -> np.ndarray:
    """Exclusive prefix sum of floor(len_i / every) (gitcode, "中间状态检查点")."""
    cu = _i64(np.asarray(cu))
    N = len(cu) - 1
    out = np.zeros(N + 1, dtype=np.int64)
    lib().oracle_checkpoint_starts(_ptr(cu), N, int(every), _ptr(out))
    return out


# --------------------------------------------------------------------------
# Exact rational form (tiny sizes only).
# --------------------------------------------------------------------------

def exact_token(q, k, v, alpha, beta, scale, S0=None):
    """One sequence, one head, exact rationals.

    q, k, v: lists of L rows of D Fractions; alpha, beta: L Fractions;
    S0: D x D Fractions as S[a][b] (keys x values) or None.
    Returns (outputs L x D, states list of S_t for t = 1..L)."""
    L, D = len(q), len(q[0])
    S = [[Fraction(0)] * D for _ in range(D)] if S0 is None else [
        list(r) for r in S0]
    outs, states = [], []
    for t in range(L):
        kS = [sum(k[t][a] * S[a][b] for a in range(D)) for b in range(D)]
        S = [[alpha[t] * (S[a][b] - beta[t] * k[t][a] * kS[b])
              + beta[t] * k[t][a] * v[t][b] for b in range(D)]
             for a in range(D)]
        outs.append([scale * sum(S[a][b] * q[t][a] for a in range(D))
                     for b in range(D)])
        states.append([row[:] for row in S])
    return outs, states


# --------------------------------------------------------------------------
# Page-3 partial transitions (tiny sizes only).
# --------------------------------------------------------------------------

def position_pair(k_i, v_i, alpha_i, beta_i):
    """The affine map S -> A S + B of one position (0539edu section 2.1's
    per-position transition pair, with the gate placement of reading R1):
    A = alpha (I - beta k k^T), B = beta k v^T.  S is keys x values."""
    k_i = np.asarray(k_i, np.float64)
    D = k_i.shape[0]
    A = alpha_i * (np.eye(D) - beta_i * np.outer(k_i, k_i))
    return A, beta_i * np.outer(k_i, np.asarray(v_i, np.float64))


def partial_transition(q, k, v, alpha, beta, scale, C, S0=None):
    """One sequence, one head, fp64 numpy, from pair composition (0539edu
    sections 2.1-2.2 and 3.2): every position is an affine pair
    (``position_pair``); inside a chunk the inclusive scan of the pairs under
    ``combine_pairs`` gives, at each position, the map from the state that
    entered the chunk to the state after that position, which the position's
    output reads; the chunk's whole composition carries the state to the next
    chunk.  Returns (out [L, D], S_final)."""
    from itertools import accumulate
    q = np.asarray(q, np.float64)
    L, D = q.shape
    S = np.zeros((D, D)) if S0 is None else np.array(S0, np.float64)
    pairs = [position_pair(k[i], v[i], alpha[i], beta[i]) for i in range(L)]
    y = np.zeros((L, D))
    for start in range(0, L, C):
        prefix = list(accumulate(pairs[start:start + C], combine_pairs))
        for i, (M, N) in enumerate(prefix, start):
            y[i] = scale * (q[i] @ (M @ S + N))
        M, N = prefix[-1]
        S = M @ S + N
    return y, S


def combine_pairs(left, right):
    """Composition of two adjacent transitions (0539edu section 2.1):
    M = M_R M_L, N = M_R N_L + N_R."""
    (ML, NL), (MR, NR) = left, right
    return MR @ ML, MR @ NL + NR
