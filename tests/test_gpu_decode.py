"""GPU parity of the decode step (one new token per sequence) against the
oracle's token recurrence over one-token sequences, through the C ABI.

The decode step is the recurrence applied once (weigao.cc "GDN 与 Chunked
Prefill", section "Prefill 和 decode 的差异"), on the state layout and pool of
the prefill (gitcode "FlashInfer GDN Prefill 完全指南", section "状态池"), so
the oracle's token form over sequences of length 1 is its definition.
"""
import numpy as np
import pytest

from gated_deltanet_chunked_varlen_amd import workloads as W
from tests import gdn_testlib as tl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _check(wl, gpu, orc):
    errs, _ = tl.compare(wl, gpu, orc)
    bars = tl.bars(wl)
    print(wl.name, {k: "%.3e" % v for k, v in errs.items()}, "bars", bars, flush=True)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])


def _dec(seed, n, dtype="bf16", hq=4, hk=4, hv=4, D=128, **kw):
    kw.setdefault("l2norm_in_kernel", True)
    kw.setdefault("init", "seq")
    kw.setdefault("init_std", 0.3)
    return W.make(seed, [1] * n, hq, hk, hv, D, dtype, **kw)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("bf16", 32),
                                     ("f16", 128), ("f16", 64),
                                     ("f32", 128), ("f32", 64), ("f32", 32)])
def test_decode_dtype_and_head_size(dtype, D):
    wl = _dec(41, 37, dtype=dtype, D=D)
    _check(wl, tl.run_gpu_decode(wl), tl.run_oracle(wl))


def test_decode_pool_in_place_16_heads():
    wl = _dec(42, 64, hq=16, hk=16, hv=16, init="pool", pool_size=128, in_place_pool=True)
    gpu = tl.run_gpu_decode(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    idx = set(int(r) for r in wl.state_indices)
    others = [r for r in range(128) if r not in idx]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


@pytest.mark.parametrize("hq,hk,hv", [(4, 2, 2), (2, 2, 6)])
def test_decode_head_sharing(hq, hk, hv):
    wl = _dec(43, 20, hq=hq, hk=hk, hv=hv)
    _check(wl, tl.run_gpu_decode(wl), tl.run_oracle(wl))


def test_decode_strided_states():
    """State views: the initial state with a non-contiguous head/row order but
    unit element stride (16-byte vector path), the final state with a
    non-unit element stride (element-by-element path)."""
    wl = _dec(46, 24, init="seq")
    H, D, N = wl.H, wl.D, wl.N
    base = torch.from_numpy(np.ascontiguousarray(
        wl.initial_state.transpose(1, 0, 2, 3))).cuda()       # [H, N, V, K]
    init = base.permute(1, 0, 2, 3)                            # [N, H, V, K] view
    outbuf = torch.zeros((H, D, D, N), dtype=torch.float32, device="cuda")
    outst = outbuf.permute(3, 0, 1, 2)                         # [N, H, V, K] view
    gpu = tl.run_gpu_decode(wl, initial_state=init, output_state=outst)
    _check(wl, dict(gpu, final=outst.cpu().numpy().astype(np.float64)), tl.run_oracle(wl))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_fp8_pool_in_place(fmt):
    wl = _dec(47, 40, init="pool", pool_size=64, in_place_pool=True,
              init_dtype=fmt, final_state_dtype=fmt)
    gpu = tl.run_gpu_decode(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    idx = set(int(r) for r in wl.state_indices)
    others = [r for r in range(64) if r not in idx]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


def test_decode_no_gates_no_state_bf16_final():
    wl = _dec(44, 9, gates=False, init=None, final_state_dtype="bf16")
    _check(wl, tl.run_gpu_decode(wl), tl.run_oracle(wl))


def test_decode_bad_state_index_sets_status_and_writes_nothing():
    wl = _dec(45, 3, init="pool", pool_size=4, in_place_pool=True)
    wl.state_indices = np.array([1, 7, 2], dtype=np.int32)   # 7 is out of range
    gpu = tl.run_gpu_decode(wl, status=True)
    assert gpu["status"] & 4
    for r in (0, 3):
        np.testing.assert_array_equal(gpu["final"][r], gpu["pool_before"][r])


def test_decode_continues_a_prefill():
    # prefill L tokens, then decode the (L+1)-th: the result is the
    # recurrence over all L+1 tokens
    L, N = 130, 3
    full = W.make(46, [L + 1] * N, 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                  init="seq", init_std=0.3)
    orc = tl.run_oracle(full)
    head = W.make(46, [L + 1] * N, 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                  init="seq", init_std=0.3)
    take = np.concatenate([np.arange(i * (L + 1), i * (L + 1) + L) for i in range(N)])
    last = np.array([i * (L + 1) + L for i in range(N)])
    head.q, head.k, head.v = full.q[take], full.k[take], full.v[take]
    head.g, head.beta = full.g[take], full.beta[take]
    head.cu_seqlens = np.arange(0, N * L + 1, L, dtype=np.int32)
    r1 = tl.run_gpu(head)
    step = W.make(46, [1] * N, 4, 4, 4, 128, "bf16", l2norm_in_kernel=True)
    step.q, step.k, step.v = full.q[last], full.k[last], full.v[last]
    step.g, step.beta = full.g[last], full.beta[last]
    step.initial_state = r1["final"].astype(np.float32)
    step.initial_state_dtype = "f32"
    r2 = tl.run_gpu_decode(step)
    assert tl.rel_l2(r2["out"], orc["out"][last]) < 2e-2
    assert tl.rel_l2(r2["final"], orc["final"]) < 2e-2
