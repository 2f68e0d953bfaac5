"""The no-allocation prefill entry point (gdn_prefill_noalloc) against the
ordinary one (gdn_prefill), both through the C ABI.

gdn_prefill_noalloc is for callers that cannot allocate device memory: the
workspace is the library's static per-GPU scratch array.  Both entry points
run the same kernels on the same inputs, so their results must agree bit for
bit; two calls in a row, the second smaller, check that the scratch left by
one call does not leak into the next.  The oracle comparison of the ordinary
entry point lives in the parity tests; here one call is also held to the
oracle's bar so that a wrong scratch address cannot pass as agreement of two
wrong results.
"""
import ctypes

import numpy as np
import pytest

from gated_deltanet_chunked_varlen_amd import _native as nat
from gated_deltanet_chunked_varlen_amd import api
from gated_deltanet_chunked_varlen_amd import workloads as W
from tests import gdn_testlib as tl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _both(wl, **extra):
    """Run ``wl`` through gdn_prefill (fresh workspace) and through
    gdn_prefill_noalloc into separate output buffers; returns both results as
    tensors."""
    d = tl.to_device(wl)
    H, D, N, T = wl.H, wl.D, wl.N, wl.T
    qdt = d["q"].dtype
    res = []
    for noalloc in (False, True):
        out = torch.full((T, H, D), float("nan"), dtype=qdt, device="cuda")
        fin = torch.full((N, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
        ck = None
        kw = dict(g=d["g"], beta=d["beta"], scale=wl.scale, cu_seqlens=d["cu_seqlens"],
                  use_qk_l2norm_in_kernel=wl.l2norm_in_kernel,
                  initial_state=d["initial_state"], output_final_state=True,
                  output=out, output_state=fin)
        if wl.checkpoint_every > 0:
            rows = int(wl.checkpoint_cu_starts[-1])
            ck = torch.full((rows, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
            kw.update(state_checkpoints=ck, checkpoint_cu_starts=d["checkpoint_cu_starts"],
                      checkpoint_every_n_tokens=wl.checkpoint_every)
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        kw["status"] = st
        kw.update(extra)
        torch.cuda.synchronize()
        if noalloc:
            before = torch.cuda.memory_allocated()
            api.chunk_gated_delta_rule_noalloc(d["q"], d["k"], d["v"], **kw)
            assert torch.cuda.memory_allocated() == before
        else:
            ws = torch.empty(api.workspace_size(api.make_params(d["q"], d["k"], d["v"], **{
                k: v for k, v in kw.items() if k != "status"})[0]),
                dtype=torch.uint8, device="cuda")
            api.chunk_gated_delta_rule(d["q"], d["k"], d["v"], workspace=ws, **kw)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        res.append((out, fin, ck))
    return res


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_prefill_on_two_calls_in_a_row(dtype):
    big = W.make(101, [700, 64, 0, 131, 1000, 65], 8, 8, 16, 128, dtype,
                 l2norm_in_kernel=True, init="seq", init_std=0.3,
                 checkpoint_every=128)
    small = W.make(102, [130, 20], 8, 8, 16, 128, dtype, l2norm_in_kernel=True,
                   init="seq", init_std=0.3)
    for wl in (big, small):
        need = api.workspace_size(api.make_params(*[tl.to_device(wl)[n] for n in ("q", "k", "v")],
                                                  cu_seqlens=tl.to_device(wl)["cu_seqlens"])[0])
        assert 0 < need <= nat.NOALLOC_SCRATCH_BYTES
        (o1, f1, c1), (o2, f2, c2) = _both(wl)
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
        if c1 is not None:
            assert torch.equal(c1, c2)
    # the second (smaller) call, no-allocation path, against the oracle
    orc = tl.run_oracle(small)
    got = dict(out=o2.float().cpu().numpy().astype(np.float64),
               final=f2.cpu().numpy().astype(np.float64), ckpt=None)
    errs, _ = tl.compare(small, got, orc)
    bars = tl.bars(small)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])


def test_noalloc_rejects_a_call_larger_than_the_scratch():
    # a shape whose workspace exceeds the scratch returns GDN_ERR_SCRATCH
    # from the host check, before anything is launched or read
    wl = W.make(103, [64], 16, 16, 16, 128, "bf16")
    d = tl.to_device(wl)
    out = torch.empty_like(d["q"])
    p, _, _ = api.make_params(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"], output=out)
    p.total_tokens = 1 << 20
    p.cu_seqlens = None
    p.num_seqs = 1
    assert api.workspace_size(p) > nat.NOALLOC_SCRATCH_BYTES
    rc = nat.lib().gdn_prefill_noalloc(ctypes.byref(p), ctypes.c_void_p(0))
    assert rc == nat.ERR_CODE["GDN_ERR_SCRATCH"]
    with pytest.raises(ValueError):
        api.chunk_gated_delta_rule_noalloc(d["q"], d["k"], d["v"])      # no output buffer


def test_noalloc_context_parallel_matches_prefill():
    # the context-parallel form takes its segment buffers from the scratch too
    wl = W.make(104, [1500, 700], 2, 2, 2, 128, "bf16", l2norm_in_kernel=True, init="seq",
                init_std=0.3)
    (o1, f1, _), (o2, f2, _) = _both(wl, use_cp=True, _cp_chunk_len=256)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
