"""Python binding of libgdn_prefill: ``chunk_gated_delta_rule``.

The call keeps the parameter names and the return convention of gitcode
"FlashInfer GDN Prefill 完全指南" (sections "API 全参数解析" and "基础用法"):
it returns ``output`` alone, or ``(output, final_state)`` when
``output_final_state`` is true; with ``state_indices`` the final state is the
caller's pool ``output_state`` itself.  The routing arguments of that API
(``use_cp``, ``_cp_chunk_len``, ``backend``) have no counterpart: there is one
implementation.

This module only marshals arguments.  torch provides device memory (outputs,
workspace) and the current stream; every step of the computation runs in the
HIP kernels of libgdn_prefill.  There is no fallback: without the built
library or a gfx950 device the call raises.
"""
from __future__ import annotations

import ctypes
from collections import OrderedDict
from typing import Optional

import torch

from . import _native as nat

_QKV_DTYPES = {torch.float32: nat.GDN_F32, torch.bfloat16: nat.GDN_BF16,
               torch.float16: nat.GDN_F16}
_STATE_DTYPES = {torch.float32: nat.GDN_F32, torch.bfloat16: nat.GDN_BF16,
                 torch.float16: nat.GDN_F16, torch.float8_e4m3fn: nat.GDN_FP8_E4M3,
                 torch.float8_e5m2: nat.GDN_FP8_E5M2}
_INDEX_TYPES = {torch.int32: nat.GDN_I32, torch.int64: nat.GDN_I64}

_VALUE_ERRORS = {"GDN_ERR_NULL", "GDN_ERR_SHAPE", "GDN_ERR_HEAD_RATIO",
                 "GDN_ERR_DTYPE", "GDN_ERR_CHECKPOINT", "GDN_ERR_STATE",
                 "GDN_ERR_MAX_SEQLEN", "GDN_ERR_WORKSPACE", "GDN_ERR_STRIDES",
                 "GDN_ERR_ALIGN", "GDN_ERR_CP", "GDN_ERR_SCRATCH"}


def _raise(rc: int):
    name = nat.ERRORS.get(rc, "GDN_ERR_%d" % rc)
    msg = "%s: %s" % (name, nat.status_string(rc))
    if name in _VALUE_ERRORS:
        raise ValueError(msg)
    if name == "GDN_ERR_DEVICE":
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, dev):
    if t is not None and (t.device != dev):
        raise ValueError("%s must be on %s" % (name, dev))


def _index(name, t):
    if t.dtype not in _INDEX_TYPES:
        raise ValueError("%s must be int32 or int64" % name)
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 1-D tensor" % name)
    return _INDEX_TYPES[t.dtype]


def _state_strides(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("states are rank-4 [rows, H, V, K]")
    return tuple(int(s) for s in t.stride())


def _broadcast(t: torch.Tensor) -> bool:
    """True when a dimension of extent > 1 has stride 0 (an expanded view):
    its elements alias, and the C ABI reads all-zero strides as
    "contiguous", so such a view must never reach it as is."""
    return any(n > 1 and st == 0 for n, st in zip(t.shape, t.stride()))


def state_tensor(name: str, t: Optional[torch.Tensor], written: bool):
    """The state tensor to hand to the library.  An expanded view (a stride
    of 0 on a dimension of extent > 1) is copied to contiguous memory when the
    library only reads it, and rejected when the library writes it."""
    if t is None or not _broadcast(t):
        return t
    if written:
        raise ValueError("%s must not be an expanded view (a stride of 0 on a "
                         "dimension of extent > 1)" % name)
    return t.contiguous()


def make_params(q, k, v, g=None, beta=None, scale=None, initial_state=None,
                output_final_state=False, cu_seqlens=None,
                use_qk_l2norm_in_kernel=False, output=None, output_state=None,
                state_checkpoints=None, checkpoint_cu_starts=None,
                checkpoint_every_n_tokens=0, state_indices=None,
                max_seqlen=None, status=None, decode=False, use_cp="auto",
                _cp_chunk_len=None):
    """Fill the C parameter block (allocates output / final state when the
    caller passes none).  Returns (params, output, output_state).  With
    ``decode`` token i is sequence i's one new token (num_seqs = T).
    ``use_cp``: "auto", True or False (context parallelism within the GPU);
    ``_cp_chunk_len``: its segment length in tokens, a multiple of 64."""
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    dev = q.device
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens),
                    ("output", output), ("output_state", output_state),
                    ("state_checkpoints", state_checkpoints),
                    ("checkpoint_cu_starts", checkpoint_cu_starts),
                    ("state_indices", state_indices), ("status", status)):
        _check_dev(name, t, dev)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [total_seq_len, heads, head_size]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if q.dtype not in _QKV_DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32, bfloat16 or float16")
    T, hq, D = q.shape
    hk, hv = k.shape[1], v.shape[1]
    if k.shape[0] != T or v.shape[0] != T or k.shape[2] != D or v.shape[2] != D:
        raise ValueError("q, k, v shapes disagree")
    H = max(hq, hv)
    p = nat.Params()
    p.total_tokens = T
    p.num_q_heads, p.num_k_heads, p.num_v_heads = hq, hk, hv
    p.head_size = D
    p.qkv_dtype = _QKV_DTYPES[q.dtype]
    p.q, p.k, p.v = _ptr(q), _ptr(k), _ptr(v)
    for name, t in (("g", g), ("beta", beta)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (T, H)
                              or not t.is_contiguous()):
            raise ValueError("%s must be contiguous float32 [%d, %d]" % (name, T, H))
    p.g, p.beta = _ptr(g), _ptr(beta)
    p.has_scale = 0 if scale is None else 1
    p.scale = 0.0 if scale is None else float(scale)
    if decode:
        if cu_seqlens is not None:
            raise ValueError("decode takes one token per sequence and no cu_seqlens")
        N = T
    elif cu_seqlens is not None:
        p.cu_seqlens_type = _index("cu_seqlens", cu_seqlens)
        p.cu_seqlens = _ptr(cu_seqlens)
        N = cu_seqlens.numel() - 1
    else:
        N = 1
    p.num_seqs = N
    p.use_qk_l2norm_in_kernel = 1 if use_qk_l2norm_in_kernel else 0
    if output is None:
        output = torch.empty((T, H, D), dtype=q.dtype, device=dev)
    elif (output.dtype != q.dtype or tuple(output.shape) != (T, H, D)
          or not output.is_contiguous()):
        raise ValueError("output must be contiguous [%d, %d, %d] %s" % (T, H, D, q.dtype))
    p.output = _ptr(output)
    if initial_state is not None:
        if initial_state.dtype not in _STATE_DTYPES:
            raise ValueError("unsupported initial_state dtype")
        initial_state = state_tensor("initial_state", initial_state, written=False)
        p.initial_state = _ptr(initial_state)
        p.initial_state_dtype = _STATE_DTYPES[initial_state.dtype]
        p.initial_state_strides = nat._i64x4(*_state_strides(initial_state))
    if state_indices is not None:
        p.state_indices_type = _index("state_indices", state_indices)
        p.state_indices = _ptr(state_indices)
        pool = output_state if output_state is not None else initial_state
        if pool is None:
            raise ValueError("state_indices needs a state pool")
        p.pool_size = pool.shape[0]
        if initial_state is not None and initial_state.shape[0] != pool.shape[0]:
            raise ValueError("initial_state and output_state pools differ in rows")
    if output_final_state:
        if output_state is None:
            if state_indices is not None:
                raise ValueError(
                    "output_state (the pool) is required with state_indices")
            output_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
        if output_state.dtype not in _STATE_DTYPES:
            raise ValueError("unsupported output_state dtype")
        output_state = state_tensor("output_state", output_state, written=True)
        p.output_final_state = 1
        p.output_state = _ptr(output_state)
        p.output_state_dtype = _STATE_DTYPES[output_state.dtype]
        p.output_state_strides = nat._i64x4(*_state_strides(output_state))
    for name, t in (("initial_state", initial_state),
                    ("output_state", output_state if output_final_state else None)):
        if t is not None:
            rows = p.pool_size if state_indices is not None else N
            if tuple(t.shape) != (rows, H, D, D):
                raise ValueError("%s must be [%d, %d, %d, %d]" % (name, rows, H, D, D))
    p.checkpoint_every_n_tokens = int(checkpoint_every_n_tokens)
    state_tensor("state_checkpoints", state_checkpoints, written=True)
    if state_checkpoints is not None:
        if state_checkpoints.dtype not in _STATE_DTYPES or not state_checkpoints.is_contiguous():
            raise ValueError("state_checkpoints must be contiguous fp32/bf16/fp16")
        if tuple(state_checkpoints.shape[1:]) != (H, D, D):
            raise ValueError("state_checkpoints must be [rows, %d, %d, %d]" % (H, D, D))
        p.state_checkpoints = _ptr(state_checkpoints)
        p.checkpoint_dtype = _STATE_DTYPES[state_checkpoints.dtype]
        p.checkpoint_rows = state_checkpoints.shape[0]
    if checkpoint_cu_starts is not None:
        p.checkpoint_cu_starts_type = _index("checkpoint_cu_starts", checkpoint_cu_starts)
        p.checkpoint_cu_starts = _ptr(checkpoint_cu_starts)
    p.max_seqlen = 0 if max_seqlen is None else int(max_seqlen)
    if isinstance(use_cp, str):
        if use_cp != "auto":
            raise ValueError('use_cp must be "auto", True or False')
        p.use_cp = nat.CP_AUTO
    else:
        p.use_cp = nat.CP_ON if use_cp else nat.CP_OFF
    p.cp_chunk_len = 0 if _cp_chunk_len is None else int(_cp_chunk_len)
    if status is not None:
        if status.dtype != torch.int32 or status.numel() < 1:
            raise ValueError("status must be an int32 tensor")
        p.status = _ptr(status)
    return p, output, output_state


def workspace_tensor(workspace: Optional[torch.Tensor], device, need: int) -> torch.Tensor:
    """The workspace a call uses: the caller's when it is a contiguous uint8
    tensor on the call's device with at least ``need`` bytes, a fresh one when
    the caller passed none or a smaller one.  Anything else raises: the
    kernels take its address as device memory of the call's device."""
    if workspace is not None:
        if (workspace.device != torch.device(device) or workspace.dtype != torch.uint8
                or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % device)
        if workspace.numel() >= need:
            return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Plan / workspace cache (gitcode "FlashInfer GDN Prefill 完全指南", section
# "内部机制：plan 缓存、地址重绑定与 CUDA Graph": the dispatcher keeps the
# shape-dependent plan and workspace and launches directly, so outputs the API
# allocates and rotating input buffers may change address without a new plan).
# Here the plan is the workspace layout the library derives from the shape on
# every call (host arithmetic only); what is worth keeping is the workspace.
# One workspace per (device, stream): calls on one stream run in order and can
# share it; calls on different streams get their own.  It grows to the largest
# call seen and is released with clear_workspace_cache().
# ---------------------------------------------------------------------------
_WS_CACHE_MAX = 64
_ws_cache: "OrderedDict[tuple, torch.Tensor]" = OrderedDict()


def cached_workspace(device, stream: int, need: int) -> torch.Tensor:
    """The cached workspace of (device, stream), grown to at least ``need``
    bytes (least recently used entries beyond 64 are dropped)."""
    dev = torch.device(device)
    key = (dev.type, dev.index, int(stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    _ws_cache.move_to_end(key)
    while len(_ws_cache) > _WS_CACHE_MAX:
        _ws_cache.popitem(last=False)
    return ws


def clear_workspace_cache() -> None:
    _ws_cache.clear()


def workspace_size(p: nat.Params) -> int:
    return int(nat.lib().gdn_prefill_workspace_size(ctypes.byref(p)))


def chunk_gated_delta_rule(q, k, v, g=None, beta=None, scale=None,
                           initial_state=None, output_final_state=False,
                           cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                           output=None, output_state=None,
                           state_checkpoints=None, checkpoint_cu_starts=None,
                           checkpoint_every_n_tokens=0, state_indices=None,
                           max_seqlen=None, status=None, workspace=None,
                           use_cp="auto", _cp_chunk_len=None):
    """Varlen chunked Gated Delta Rule prefill on the current stream.

    Shapes: q [T, hq, D], k [T, hk, D], v [T, hv, D] (float32 or bfloat16);
    g, beta [T, H] float32 (H = max(hq, hv)); cu_seqlens [N+1] int32/int64;
    states [N or pool, H, D(v), D(k)].  ``status`` (optional int32 device
    tensor) receives the device-side check bits.  ``workspace`` (optional
    uint8 device tensor) is used instead of the workspace cached for the
    current (device, stream).  ``use_cp`` ("auto", True, False) and
    ``_cp_chunk_len`` (tokens, a multiple of 64) control context parallelism
    within the GPU (gitcode "FlashInfer GDN Prefill 完全指南", sections "API
    全参数解析" and "Cake GDN CP 后端"); True outside its domain (bf16 / fp16
    inputs, head size 128, at most 63 sequences) raises.
    """
    lib = nat.lib()
    p, output, output_state = make_params(
        q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
        use_qk_l2norm_in_kernel, output, output_state, state_checkpoints,
        checkpoint_cu_starts, checkpoint_every_n_tokens, state_indices,
        max_seqlen, status, use_cp=use_cp, _cp_chunk_len=_cp_chunk_len)
    need = int(lib.gdn_prefill_workspace_size(ctypes.byref(p)))
    if need == 0:
        rc = lib.gdn_validate_host(ctypes.byref(p))
        _raise(rc if rc != 0 else nat.ERR_CODE["GDN_ERR_SHAPE"])
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if workspace is None and torch.cuda.is_current_stream_capturing():
            # a graph keeps the address it was captured with: give it memory of
            # its own capture pool rather than the shared cached workspace
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif workspace is None:
            workspace = cached_workspace(q.device, stream, need)
        else:
            workspace = workspace_tensor(workspace, q.device, need)
        p.workspace = ctypes.c_void_p(workspace.data_ptr())
        p.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.gdn_prefill(ctypes.byref(p), ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if output_final_state:
        return output, output_state
    return output


def chunk_gated_delta_rule_noalloc(q, k, v, g=None, beta=None, scale=None,
                                   initial_state=None, output_final_state=False,
                                   cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                                   output=None, output_state=None,
                                   state_checkpoints=None, checkpoint_cu_starts=None,
                                   checkpoint_every_n_tokens=0, state_indices=None,
                                   max_seqlen=None, status=None, use_cp="auto",
                                   _cp_chunk_len=None):
    """``chunk_gated_delta_rule`` through gdn_prefill_noalloc: the library's
    static device scratch (128 MiB per GPU) serves as the workspace and
    nothing is allocated, here or in the library.  ``output`` (and
    ``output_state`` with ``output_final_state``) must be given, and an
    expanded ``initial_state`` is refused rather than copied.  Calls that
    overlap in time on one GPU race on the shared scratch."""
    if output is None:
        raise ValueError("the no-allocation call needs an output buffer")
    if output_final_state and output_state is None:
        raise ValueError("the no-allocation call needs an output_state buffer")
    if initial_state is not None and _broadcast(initial_state):
        raise ValueError("initial_state must not be an expanded view here")
    lib = nat.lib()
    p, output, output_state = make_params(
        q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
        use_qk_l2norm_in_kernel, output, output_state, state_checkpoints,
        checkpoint_cu_starts, checkpoint_every_n_tokens, state_indices,
        max_seqlen, status, use_cp=use_cp, _cp_chunk_len=_cp_chunk_len)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gdn_prefill_noalloc(ctypes.byref(p), ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if output_final_state:
        return output, output_state
    return output


def gated_delta_rule_decode(q, k, v, g=None, beta=None, scale=None,
                            initial_state=None, output_final_state=True,
                            use_qk_l2norm_in_kernel=False, output=None,
                            output_state=None, state_indices=None, status=None):
    """One decode step: token i of q/k/v [N, heads, D] is the new token of
    sequence i; g, beta [N, H].  The state pool semantics are those of
    ``chunk_gated_delta_rule`` (with ``state_indices`` the final state is the
    pool ``output_state``; it may be ``initial_state`` itself).  Returns
    ``output`` [N, H, D], or ``(output, final_state)``."""
    lib = nat.lib()
    p, output, output_state = make_params(
        q, k, v, g, beta, scale, initial_state, output_final_state, None,
        use_qk_l2norm_in_kernel, output, output_state, None, None, 0,
        state_indices, None, status, decode=True)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gdn_decode(ctypes.byref(p), ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if output_final_state:
        return output, output_state
    return output


def build_chunk_indices(cu_seqlens: Optional[torch.Tensor], total_tokens: int,
                        device=None):
    """The device-side chunk-index builder alone.  Returns (chunk_indices
    [cap, 2], cu_chunks [N+1], seq_starts [N+1], n_chunks [1], status [1]),
    all int32 device tensors, computed without any host synchronisation."""
    lib = nat.lib()
    if cu_seqlens is not None:
        device = cu_seqlens.device
        ctype = _index("cu_seqlens", cu_seqlens)
        N = cu_seqlens.numel() - 1
    else:
        ctype, N = nat.GDN_I32, 1
    cap = int(lib.gdn_max_chunks(int(total_tokens), int(N)))
    i32 = dict(dtype=torch.int32, device=device)
    table = torch.empty((max(cap, 1), 2), **i32)
    cu_chunks = torch.empty(N + 1, **i32)
    starts = torch.empty(N + 1, **i32)
    n = torch.empty(1, **i32)
    st = torch.empty(1, **i32)
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
        rc = lib.gdn_build_chunk_indices(
            _ptr(cu_seqlens), ctype, N, int(total_tokens), _ptr(table),
            _ptr(cu_chunks), _ptr(starts), _ptr(n), _ptr(st),
            ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return table[:cap], cu_chunks, starts, n, st


# ---------------------------------------------------------------------------
# Graph replay with rotating buffers (gitcode, section "内部机制：plan 缓存、
# 地址重绑定与 CUDA Graph": fixed-address prepared calls replay from a CUDA
# graph, captured on the first call only).  A captured graph holds the
# addresses it was captured with, so this cache keeps one executable graph per
# address set: a caller that rotates among a few sets of q/k/v/output buffers
# (double or triple buffering) captures each set once and replays it after.
# Metadata needs no host-side resolution before capture: the chunk table is
# built on the device inside the call.
# ---------------------------------------------------------------------------
class PrefillGraphs:
    """``chunk_gated_delta_rule`` through HIP graphs, one per distinct set of
    tensor addresses and sizes (at most ``max_graphs``, least recently used
    dropped).  Call it with the arguments of ``chunk_gated_delta_rule``;
    ``output`` (and ``output_state`` with ``output_final_state``) must be
    given, since a replay writes into the buffers it was captured with.  The
    first call with a new address set runs the call once eagerly (on a side
    stream, to load the library and build its workspace) and captures it;
    every call replays the graph of its address set on the current stream.
    ``graphs_captured`` counts captures."""

    def __init__(self, max_graphs: int = 16):
        self.max_graphs = max_graphs
        self._graphs: "OrderedDict[tuple, tuple]" = OrderedDict()
        self.graphs_captured = 0

    @staticmethod
    def _key(args, kwargs):
        parts = []
        for x in list(args) + [kwargs[k] for k in sorted(kwargs)]:
            if isinstance(x, torch.Tensor):
                parts.append(("t", x.data_ptr(), tuple(x.shape), tuple(x.stride()), str(x.dtype),
                              str(x.device)))
            else:
                parts.append(("v", repr(x)))
        return tuple(sorted(kwargs)), tuple(parts)

    def __call__(self, *args, **kwargs):
        if kwargs.get("output") is None:
            raise ValueError("PrefillGraphs needs an explicit output buffer")
        if kwargs.get("output_final_state") and kwargs.get("output_state") is None:
            raise ValueError("PrefillGraphs needs an explicit output_state buffer")
        if len(args) > 18:
            raise ValueError("pass workspace by keyword")
        kwargs = {k: v for k, v in kwargs.items() if k != "workspace"}
        key = self._key(args, kwargs)
        hit = self._graphs.get(key)
        if hit is None:
            # each graph owns its workspace, so graphs of different address
            # sets and eager calls never share one
            p, _, _ = make_params(*args, **kwargs)
            ws = torch.empty(max(workspace_size(p), 1), dtype=torch.uint8,
                             device=args[0].device)
            kwargs_ws = dict(kwargs, workspace=ws)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                chunk_gated_delta_rule(*args, **kwargs_ws)
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                res = chunk_gated_delta_rule(*args, **kwargs_ws)
            hit = (graph, res, ws)
            self._graphs[key] = hit
            self.graphs_captured += 1
            while len(self._graphs) > self.max_graphs:
                self._graphs.popitem(last=False)
        self._graphs.move_to_end(key)
        graph, res, _ = hit
        graph.replay()
        return res
