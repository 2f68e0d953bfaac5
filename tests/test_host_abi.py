"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and its host-side checks return the documented codes.  No compute
call is made (no GPU here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "gdn_prefill.h")


def _lib():
    from gated_deltanet_chunked_varlen_amd import _native
    return _native


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(gdn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    nat = _lib()
    L = nat.lib()
    declared = declared_functions()
    assert set(declared) == set(nat.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", nat.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    assert set(declared) <= exported


def test_abi_version_and_strings():
    nat = _lib()
    assert nat.lib().gdn_abi_version() == 2
    for code in list(nat.ERRORS) + [1, 2, 4, 8]:
        assert nat.status_string(code) != "unknown code"


@pytest.mark.parametrize("T,N,want", [
    (0, 3, 0), (128, 1, 2), (130, 1, 3), (515, 6, 13), (4096, 2, 65),
    (262144, 1, 4096), (5, 10, 5)])
def test_max_chunks_bound(T, N, want):
    assert _lib().lib().gdn_max_chunks(T, N) == want


def test_max_chunks_bounds_every_batch():
    from oracle import oracle
    L = _lib().lib()
    rng = np.random.default_rng(0)
    for _ in range(200):
        N = int(rng.integers(1, 12))
        lens = rng.integers(0, 300, N)
        lens[rng.random(N) < 0.3] = 0
        cu = np.concatenate([[0], np.cumsum(lens)])
        n = oracle.chunk_table(cu, 64)[2]
        assert n <= L.gdn_max_chunks(int(cu[-1]), N)


def _params(**kw):
    nat = _lib()
    p = nat.Params()
    p.total_tokens = kw.get("T", 128)
    p.num_seqs = kw.get("N", 1)
    p.num_q_heads = kw.get("hq", 4)
    p.num_k_heads = kw.get("hk", 4)
    p.num_v_heads = kw.get("hv", 4)
    p.head_size = kw.get("D", 128)
    p.qkv_dtype = kw.get("dtype", nat.GDN_BF16)
    fake = ctypes.c_void_p(0x1000)
    p.q = p.k = p.v = p.output = fake
    p.cu_seqlens = fake if kw.get("cu", True) else None
    p.cu_seqlens_type = nat.GDN_I32
    for f, v in kw.get("extra", {}).items():
        setattr(p, f, v)
    return p


def _validate(p, with_ws=True):
    nat = _lib()
    L = nat.lib()
    if with_ws:
        need = L.gdn_prefill_workspace_size(ctypes.byref(p))
        p.workspace = ctypes.c_void_p(0x2000)
        p.workspace_bytes = need
    return L.gdn_validate_host(ctypes.byref(p))


def code(name):
    return _lib().ERR_CODE[name]


def test_validate_ok_and_workspace():
    nat = _lib()
    p = _params(T=4096, N=2, hq=16, hk=16, hv=16)
    assert _validate(p) == 0
    need = nat.lib().gdn_prefill_workspace_size(ctypes.byref(p))
    # 65 chunks x 16 heads x (W, Ktilde, U, q fragments: 4 blocks of 64x128,
    # masked Q K^T: 64x64) in bf16 + G
    assert need >= 65 * 16 * (4 * 64 * 128 * 2 + 64 * 64 * 2 + 64 * 4)
    p32 = _params(T=4096, N=2, hq=16, hk=16, hv=16, dtype=nat.GDN_F32)
    need32 = nat.lib().gdn_prefill_workspace_size(ctypes.byref(p32))
    # fp32: W, Ktilde, U, N (4 blocks of 64x128) + chunk-start states 128x128
    assert need32 >= 65 * 16 * (4 * 64 * 128 * 4 + 128 * 128 * 4 + 64 * 4)
    p.workspace_bytes = need - 1
    assert nat.lib().gdn_validate_host(ctypes.byref(p)) == code("GDN_ERR_WORKSPACE")
    # the workspace must start on a 256-byte boundary
    p.workspace_bytes = need
    p.workspace = ctypes.c_void_p(0x2010)
    assert nat.lib().gdn_validate_host(ctypes.byref(p)) == code("GDN_ERR_ALIGN")


@pytest.mark.parametrize("kw,err", [
    (dict(D=96), "GDN_ERR_SHAPE"),
    (dict(T=-1), "GDN_ERR_SHAPE"),
    (dict(N=2, cu=False), "GDN_ERR_SHAPE"),
    (dict(hq=4, hk=2, hv=4), "GDN_ERR_HEAD_RATIO"),
    (dict(hq=4, hk=4, hv=6), "GDN_ERR_HEAD_RATIO"),
    (dict(dtype=7), "GDN_ERR_DTYPE"),
    (dict(dtype=3), "GDN_ERR_DTYPE"),           # 8-bit floats are for states only
    (dict(extra=dict(q=None)), "GDN_ERR_NULL"),
    (dict(extra=dict(q=ctypes.c_void_p(0x1008))), "GDN_ERR_ALIGN"),
    (dict(extra=dict(output=ctypes.c_void_p(0x1004))), "GDN_ERR_ALIGN"),
    (dict(extra=dict(checkpoint_every_n_tokens=100,
                     state_checkpoints=ctypes.c_void_p(8),
                     checkpoint_cu_starts=ctypes.c_void_p(8))), "GDN_ERR_CHECKPOINT"),
    (dict(extra=dict(checkpoint_every_n_tokens=64,
                     state_checkpoints=ctypes.c_void_p(8))), "GDN_ERR_CHECKPOINT"),
    (dict(extra=dict(checkpoint_every_n_tokens=64)), "GDN_ERR_CHECKPOINT"),
    (dict(extra=dict(output_final_state=1)), "GDN_ERR_STATE"),
    (dict(extra=dict(state_indices=ctypes.c_void_p(8), pool_size=0)), "GDN_ERR_STATE"),
    (dict(T=100, N=4, extra=dict(max_seqlen=24)), "GDN_ERR_MAX_SEQLEN"),
    (dict(T=100, N=4, extra=dict(max_seqlen=101)), "GDN_ERR_MAX_SEQLEN"),
    (dict(extra=dict(max_seqlen=-1)), "GDN_ERR_MAX_SEQLEN"),
])
def test_validate_errors(kw, err):
    assert _validate(_params(**kw)) == code(err)


def test_validate_accepts_legal_variants():
    nat = _lib()
    assert _validate(_params(hq=8, hk=4, hv=4)) == 0           # GQA
    assert _validate(_params(hq=4, hk=4, hv=12)) == 0          # GVA
    assert _validate(_params(T=100, N=4, extra=dict(max_seqlen=25))) == 0
    assert _validate(_params(T=0, N=3)) == 0                    # empty batch
    assert _validate(_params(dtype=nat.GDN_F32, D=32)) == 0
    assert _validate(_params(dtype=nat.GDN_F16, D=64)) == 0     # fp16 inputs


def test_validate_strides():
    nat = _lib()
    H, D, N = 4, 128, 1
    ok = nat._i64x4(H * D * D, D * D, D, 1)
    transposed = nat._i64x4(H * D * D, D * D, 1, D)
    overlap = nat._i64x4(H * D * D, D, D, 1)
    negative = nat._i64x4(H * D * D, D * D, D, -1)
    for strides, want in ((ok, 0), (transposed, 0),
                          (overlap, code("GDN_ERR_STRIDES")),
                          (negative, code("GDN_ERR_STRIDES"))):
        p = _params(extra=dict(initial_state=ctypes.c_void_p(8),
                               initial_state_dtype=nat.GDN_F32,
                               initial_state_strides=strides))
        assert _validate(p) == want


def test_state_dtypes_accepted_and_rejected():
    """All five state types are accepted for initial, final and checkpoint
    states; anything else is GDN_ERR_DTYPE."""
    nat = _lib()
    for dt in (nat.GDN_F32, nat.GDN_BF16, nat.GDN_F16, nat.GDN_FP8_E4M3, nat.GDN_FP8_E5M2):
        p = _params(extra=dict(initial_state=ctypes.c_void_p(8), initial_state_dtype=dt,
                               output_final_state=1, output_state=ctypes.c_void_p(8),
                               output_state_dtype=dt))
        assert _validate(p) == 0, dt
    for bad in (5, -1):
        p = _params(extra=dict(initial_state=ctypes.c_void_p(8), initial_state_dtype=bad))
        assert _validate(p) == code("GDN_ERR_DTYPE")
        p = _params(extra=dict(output_final_state=1, output_state=ctypes.c_void_p(8),
                               output_state_dtype=bad))
        assert _validate(p) == code("GDN_ERR_DTYPE")


def test_workspace_size_zero_for_bad_shape():
    nat = _lib()
    p = _params(D=48)
    assert nat.lib().gdn_prefill_workspace_size(ctypes.byref(p)) == 0


def _validate_decode(p):
    return _lib().lib().gdn_validate_decode_host(ctypes.byref(p))


def test_validate_decode_ok():
    assert _validate_decode(_params(T=64, N=64, cu=False)) == 0
    assert _validate_decode(_params(T=0, N=0, cu=False)) == 0
    assert _validate_decode(_params(T=8, N=8, cu=False, hq=8, hk=4, hv=4)) == 0


@pytest.mark.parametrize("kw,err", [
    (dict(T=64, N=32, cu=False), "GDN_ERR_SHAPE"),        # one token per sequence
    (dict(T=8, N=8, cu=True), "GDN_ERR_SHAPE"),           # no cu_seqlens
    (dict(T=8, N=8, cu=False, D=48), "GDN_ERR_SHAPE"),
    (dict(T=8, N=8, cu=False, hq=4, hk=2, hv=4), "GDN_ERR_HEAD_RATIO"),
    (dict(T=8, N=8, cu=False, dtype=3), "GDN_ERR_DTYPE"),
    (dict(T=8, N=8, cu=False, extra=dict(checkpoint_every_n_tokens=64)), "GDN_ERR_CHECKPOINT"),
    (dict(T=8, N=8, cu=False, extra=dict(output_final_state=1)), "GDN_ERR_STATE"),
    (dict(T=8, N=8, cu=False, extra=dict(k=None)), "GDN_ERR_NULL"),
    (dict(T=8, N=8, cu=False, extra=dict(v=ctypes.c_void_p(0x1002))), "GDN_ERR_ALIGN"),
])
def test_validate_decode_errors(kw, err):
    assert _validate_decode(_params(**kw)) == code(err)


# ------------------------------------------------ binding argument checks

def test_expanded_states_are_copied_or_rejected():
    """An expanded state view (stride 0 on a dimension of extent > 1) aliases
    its elements and would read as "contiguous" through the C ABI: a state the
    library only reads is copied to contiguous memory first, one it writes is
    refused before any launch."""
    torch = pytest.importorskip("torch")
    from gated_deltanet_chunked_varlen_amd import api
    base = torch.zeros(())
    view = base.expand(3, 2, 32, 32)
    assert view.stride() == (0, 0, 0, 0)
    got = api.state_tensor("initial_state", view, written=False)
    assert got.is_contiguous() and got.stride() == (2048, 1024, 32, 1)
    with pytest.raises(ValueError):
        api.state_tensor("output_state", view, written=True)
    # one broadcast dimension is enough
    part = torch.zeros(1, 2, 32, 32).expand(4, 2, 32, 32)
    with pytest.raises(ValueError):
        api.state_tensor("state_checkpoints", part, written=True)
    # ordinary, permuted and extent-1 zero-stride views pass through as they are
    plain = torch.zeros(3, 2, 32, 32)
    assert api.state_tensor("output_state", plain, written=True) is plain
    perm = torch.zeros(2, 3, 32, 32).permute(1, 0, 2, 3)
    assert api.state_tensor("output_state", perm, written=True) is perm
    one = torch.zeros(1, 2, 32, 32).expand(1, 2, 32, 32)
    assert api.state_tensor("output_state", one, written=True) is one


def test_workspace_argument_checked():
    torch = pytest.importorskip("torch")
    from gated_deltanet_chunked_varlen_amd import api
    ws = torch.zeros(100, dtype=torch.uint8)
    assert api.workspace_tensor(ws, "cpu", 64) is ws
    fresh = api.workspace_tensor(ws, "cpu", 256)        # too small: a new one
    assert fresh is not ws and fresh.numel() == 256
    with pytest.raises(ValueError):
        api.workspace_tensor(torch.zeros(100, dtype=torch.float32), "cpu", 64)
    with pytest.raises(ValueError):
        api.workspace_tensor(torch.zeros(200, dtype=torch.uint8)[::2], "cpu", 64)
    with pytest.raises(ValueError):
        api.workspace_tensor(ws, "meta", 64)            # another device


def test_noalloc_host_checks_without_a_device():
    # gdn_prefill_noalloc refuses a NULL parameter block and a call whose
    # workspace exceeds its static scratch before it touches the GPU
    nat = _lib()
    L = nat.lib()
    assert L.gdn_prefill_noalloc(None, None) == nat.ERR_CODE["GDN_ERR_NULL"]
    p = nat.Params()
    p.total_tokens, p.num_seqs = 1 << 20, 1
    p.num_q_heads = p.num_k_heads = p.num_v_heads = 16
    p.head_size = 128
    p.qkv_dtype = 1
    assert L.gdn_prefill_workspace_size(ctypes.byref(p)) > nat.NOALLOC_SCRATCH_BYTES
    assert L.gdn_prefill_noalloc(ctypes.byref(p), None) == nat.ERR_CODE["GDN_ERR_SCRATCH"]
    p.head_size = 48
    assert L.gdn_prefill_noalloc(ctypes.byref(p), None) == nat.ERR_CODE["GDN_ERR_SHAPE"]


def test_params_struct_layout_matches_the_header():
    # the ctypes view against offsetof / sizeof from a C compiler reading
    # include/gdn_prefill.h
    import tempfile
    nat = _lib()
    fields = [f for f, _ in nat.Params._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>',
           '#include "%s"' % os.path.join(ROOT, "include", "gdn_prefill.h"),
           "int main(void) {",
           '  printf("%zu\\n", sizeof(gdn_prefill_params));']
    src += ['  printf("%%zu\\n", offsetof(gdn_prefill_params, %s));' % f for f in fields]
    src += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.check_call(["gcc", "-std=c99", c, "-o", exe])
        got = [int(x) for x in subprocess.check_output([exe]).split()]
    assert got[0] == ctypes.sizeof(nat.Params)
    assert got[1:] == [getattr(nat.Params, f).offset for f in fields]


def test_context_parallel_arguments_checked():
    nat = _lib()
    L = nat.lib()
    assert _validate(_params(T=8192, N=1, hq=2, hk=2, hv=2, cu=False,
                             extra=dict(use_cp=nat.CP_ON))) == 0
    assert _validate(_params(extra=dict(use_cp=3))) == code("GDN_ERR_CP")
    assert _validate(_params(extra=dict(use_cp=-1))) == code("GDN_ERR_CP")
    assert _validate(_params(extra=dict(cp_chunk_len=100))) == code("GDN_ERR_CP")
    assert _validate(_params(extra=dict(cp_chunk_len=-64))) == code("GDN_ERR_CP")
    # on, outside the domain: head size 64, fp32 inputs, more than 63 sequences
    assert _validate(_params(D=64, extra=dict(use_cp=nat.CP_ON))) == code("GDN_ERR_CP")
    assert _validate(_params(dtype=nat.GDN_F32, extra=dict(use_cp=nat.CP_ON))) == code("GDN_ERR_CP")
    assert _validate(_params(T=6400, N=100, extra=dict(use_cp=nat.CP_ON))) == code("GDN_ERR_CP")
    # auto, off and the segment length move the workspace: a long call with
    # two heads takes CP under auto (fp32 start states, local states and
    # transitions, [N][segments][H][D][D] each)
    ws = lambda **e: L.gdn_prefill_workspace_size(ctypes.byref(
        _params(T=16384, N=1, hq=2, hk=2, hv=2, cu=False, extra=e)))
    base = ws(use_cp=nat.CP_OFF)
    assert ws(use_cp=nat.CP_AUTO) > base
    assert ws(use_cp=nat.CP_ON, cp_chunk_len=1024) == base + 3 * 16 * 2 * 128 * 128 * 4
    # a batch that fills the GPU stays on the ordinary pass under auto
    big = lambda **e: L.gdn_prefill_workspace_size(ctypes.byref(
        _params(T=4096, N=2, hq=16, hk=16, hv=16, extra=e)))
    assert big(use_cp=nat.CP_AUTO) == big(use_cp=nat.CP_OFF)


def test_shared_k_and_q_fragments_sized_per_source_head():
    # 16-bit inputs keep the normalised k and q fragments once per (chunk, k
    # head) and (chunk, q head): a GVA call with 16 q/k heads and 32 v heads
    # needs 2 x 16 fewer 64 x D blocks per chunk than one with 32 of each
    nat = _lib()
    L = nat.lib()
    ws = lambda hq, hk, hv: L.gdn_prefill_workspace_size(ctypes.byref(
        _params(T=4096, N=2, hq=hq, hk=hk, hv=hv, extra=dict(use_cp=nat.CP_OFF))))
    cap = L.gdn_max_chunks(4096, 2)
    assert ws(32, 32, 32) - ws(16, 16, 32) == 2 * 16 * cap * 64 * 128 * 2
    # fp32 inputs keep Ktilde per sab head (no q fragments)
    ws32 = lambda hq, hk, hv: L.gdn_prefill_workspace_size(ctypes.byref(
        _params(T=4096, N=2, hq=hq, hk=hk, hv=hv, dtype=nat.GDN_F32)))
    assert ws32(32, 32, 32) == ws32(16, 16, 32)
