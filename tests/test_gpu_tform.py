"""GPU parity of the state pass in its T form, through the C ABI.

16-bit calls at D = 128 without context parallelism take the T form where
the state pass runs two or four 16-column tiles per workgroup, or where the
intermediates outgrow the last-level cache: the intra-chunk pass stores
-T diag(beta) (T = (I + A)^-1) and two row scales instead of -W, Ktilde^T
and U, and the state pass forms N = U - W S =
(-T diag(beta)) (diag(exp(G) / |k|) (K S) - V) and
Ktilde^T N = K^T diag(exp(G_last - G) / |k|) N from the raw k and v rows
(0539edu "GDN与线性注意力GPU并行实现", section 3.2: W and U are T applied to
the decayed keys and the values, so the products can take T last; weigao.cc
"GDN 与 Chunked Prefill", the WY form).  The oracle's token recurrence is
still the definition.  The cases cover four, two and one tile per workgroup,
ragged lengths with empty, one-token and chunk-boundary sequences,
checkpoints, in-place pools, shared q/k heads, fp16, narrow states and inputs
normalised outside the kernel.
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


def _tiles_per_cu(wl):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return wl.N * wl.H * (wl.D // 16) / cus


def _four_tiles(wl):
    return wl.D == 128 and _tiles_per_cu(wl) >= 4


def _lengths(seed, n, hi):
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, hi, size=n)]
    lengths[:6] = [0, 1, 64, 65, 127, 128]
    return lengths


def _check(wl, gpu, orc):
    errs, _ = tl.compare(wl, gpu, orc)
    bars = tl.bars(wl)
    print(wl.name, {k: "%.3e" % v for k, v in errs.items()}, "bars", bars, flush=True)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])


CASES = {
    "bf16_equal_heads_ckpt": dict(heads=(8, 8, 8), dtype="bf16", l2norm_in_kernel=True,
                                  init="seq", checkpoint_every=128),
    "f16_equal_heads": dict(heads=(8, 8, 8), dtype="f16", l2norm_in_kernel=True, init="seq",
                            init_dtype="f16", final_state_dtype="f16"),
    "bf16_gva_pool": dict(heads=(4, 4, 8), dtype="bf16", l2norm_in_kernel=True, init="pool",
                          pool_size=70, in_place_pool=True),
    "bf16_gqa_norm_outside": dict(heads=(8, 2, 2), dtype="bf16", normalise_in_generator=True,
                                  init="seq", checkpoint_every=64, checkpoint_dtype="bf16"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_tform_four_tile_pass(case):
    kw = dict(CASES[case])
    hq, hk, hv = kw.pop("heads")
    dtype = kw.pop("dtype")
    seed = 60 + sorted(CASES).index(case)
    H = max(hq, hk, hv)
    n = -(-1024 // (8 * H)) + 3
    wl = W.make(seed, _lengths(seed, n, 300), hq, hk, hv, 128, dtype, name="tform_" + case,
                init_std=0.3, **kw)
    assert _four_tiles(wl)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    if kw.get("in_place_pool"):
        rows = set(int(r) for r in wl.state_indices)
        others = [r for r in range(kw["pool_size"]) if r not in rows]
        np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


def test_tform_long_sequences_large_keys():
    # unnormalised keys of norm ~45 (normalised in the kernel) and long
    # sequences: the raw k rows enter K S unscaled, 1/|k| is applied after
    wl = W.make(66, [3000, 2500] + [200] * 14, 8, 8, 8, 128, "bf16", l2norm_in_kernel=True,
                init="seq", init_std=0.3, name="tform_large_keys")
    wl.k = wl.k * 4.0          # a power of two: still exact in bf16
    assert _four_tiles(wl)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_tform_two_tile_pass():
    # between one and four tiles per CU: two tiles per workgroup
    wl = W.make(67, _lengths(67, 10, 400), 8, 8, 8, 128, "bf16", l2norm_in_kernel=True,
                init="pool", pool_size=23, in_place_pool=True, init_std=0.3,
                checkpoint_every=192, name="tform_two_tiles")
    assert 1 < _tiles_per_cu(wl) < 4
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_tform_one_tile_pass_large_call():
    # one 65 536-token sequence with four heads without context parallelism:
    # one tile per workgroup, intermediates past the last-level cache
    wl = W.long_l65536_h4_d128()
    assert _tiles_per_cu(wl) <= 1
    gpu = tl.run_gpu(wl, status=True, use_cp=False)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
