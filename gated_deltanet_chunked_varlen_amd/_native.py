"""ctypes view of libgdn_prefill (include/gdn_prefill.h).

Argument marshalling only: no arithmetic of the method happens in Python.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_PREFILL_LIB names another build of the library (e.g. one whose host
# code carries sanitizers); the default is the in-tree build
LIB_PATH = os.environ.get("GDN_PREFILL_LIB") or os.path.join(HERE, "libgdn_prefill.so")

GDN_F32, GDN_BF16, GDN_F16, GDN_FP8_E4M3, GDN_FP8_E5M2 = 0, 1, 2, 3, 4
GDN_I32, GDN_I64 = 0, 1

GDN_OK = 0
ERRORS = {
    -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_HEAD_RATIO",
    -4: "GDN_ERR_DTYPE", -5: "GDN_ERR_CHECKPOINT", -6: "GDN_ERR_STATE",
    -7: "GDN_ERR_MAX_SEQLEN", -8: "GDN_ERR_WORKSPACE", -9: "GDN_ERR_STRIDES",
    -10: "GDN_ERR_DEVICE", -11: "GDN_ERR_LAUNCH", -12: "GDN_ERR_ALIGN",
    -13: "GDN_ERR_SCRATCH", -14: "GDN_ERR_CP",
}
NOALLOC_SCRATCH_BYTES = 128 << 20
CP_AUTO, CP_ON, CP_OFF = 0, 1, 2
ABI_VERSION = 2
ERR_CODE = {v: k for k, v in ERRORS.items()}
STATUS_CU_SEQLENS = 1
STATUS_CHECKPOINT_STARTS = 2
STATUS_STATE_INDEX = 4
STATUS_CHUNK_CAPACITY = 8

# every symbol include/gdn_prefill.h declares
EXPORTS = [
    "gdn_abi_version", "gdn_status_string", "gdn_max_chunks",
    "gdn_prefill_workspace_size", "gdn_validate_host", "gdn_prefill",
    "gdn_prefill_timed", "gdn_build_chunk_indices", "gdn_decode",
    "gdn_validate_decode_host", "gdn_prefill_noalloc",
]

_i64x4 = ctypes.c_int64 * 4


class Params(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("has_scale", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("cu_seqlens", ctypes.c_void_p),
        ("cu_seqlens_type", ctypes.c_int32),
        ("use_qk_l2norm_in_kernel", ctypes.c_int32),
        ("output", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("initial_state_dtype", ctypes.c_int32),
        ("initial_state_strides", _i64x4),
        ("output_final_state", ctypes.c_int32),
        ("output_state", ctypes.c_void_p),
        ("output_state_dtype", ctypes.c_int32),
        ("output_state_strides", _i64x4),
        ("state_indices", ctypes.c_void_p),
        ("state_indices_type", ctypes.c_int32),
        ("pool_size", ctypes.c_int64),
        ("checkpoint_every_n_tokens", ctypes.c_int32),
        ("state_checkpoints", ctypes.c_void_p),
        ("checkpoint_dtype", ctypes.c_int32),
        ("checkpoint_rows", ctypes.c_int64),
        ("checkpoint_cu_starts", ctypes.c_void_p),
        ("checkpoint_cu_starts_type", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int64),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("status", ctypes.c_void_p),
        ("use_cp", ctypes.c_int32),
        ("cp_chunk_len", ctypes.c_int64),
    ]


_lib = None


def lib():
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libgdn_prefill.so is not built; run "
                "`python -m gated_deltanet_chunked_varlen_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_abi_version.argtypes = []
        if L.gdn_abi_version() != ABI_VERSION:
            raise ImportError("libgdn_prefill.so has ABI version %d, this binding expects %d; "
                              "rebuild it" % (L.gdn_abi_version(), ABI_VERSION))
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_max_chunks.restype = ctypes.c_int64
        L.gdn_max_chunks.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.gdn_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(Params)]
        L.gdn_validate_host.restype = ctypes.c_int
        L.gdn_validate_host.argtypes = [ctypes.POINTER(Params)]
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_prefill.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p]
        L.gdn_prefill_timed.restype = ctypes.c_int
        L.gdn_prefill_timed.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p,
                                        ctypes.c_void_p * 5]
        L.gdn_prefill_noalloc.restype = ctypes.c_int
        L.gdn_prefill_noalloc.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p]
        L.gdn_decode.restype = ctypes.c_int
        L.gdn_decode.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p]
        L.gdn_validate_decode_host.restype = ctypes.c_int
        L.gdn_validate_decode_host.argtypes = [ctypes.POINTER(Params)]
        L.gdn_build_chunk_indices.restype = ctypes.c_int
        L.gdn_build_chunk_indices.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().gdn_status_string(int(code)).decode()
