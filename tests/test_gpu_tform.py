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


def test_tform_one_tile_pass_ragged_sequences_with_warmup():
    # two sequences of 39 963 and 25 541 tokens (ragged last chunks), four
    # heads: one tile per workgroup with the intermediates past the
    # last-level cache, so the L2 warm-up wave runs, clamping the rows of
    # each sequence's last chunk like the loaders
    wl = W.make(71, [39963, 25541], 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                init="seq", init_std=0.3, checkpoint_every=4096,
                name="tform_one_tile_ragged")
    assert _tiles_per_cu(wl) <= 1
    gpu = tl.run_gpu(wl, status=True, use_cp=False)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def _align(x):
    return (x + 255) // 256 * 256


def tform_workspace_offsets(T, N, H, D, hq, hk):
    """Byte offsets of the factor blocks (in the W region) and of the row
    scales in a 16-bit call's workspace (the layout of
    gdn_prefill_workspace_size: chunk tables, W, k fragments per k head, U,
    q fragments per q head, P, gates, row scales, each 256-byte aligned)."""
    from gated_deltanet_chunked_varlen_amd import _native as nat
    cap = int(nat.lib().gdn_max_chunks(T, N))
    blocks = cap * H
    sizes = [8 * max(cap, 1), 8 * max(cap, 1), 4 * (N + 1), 4 * (N + 1), 4]
    off = 0
    for sz in sizes:
        off = _align(off + sz)
    wf = off
    after = [blocks * 64 * D * 2, cap * hk * 64 * D * 2, blocks * 64 * D * 2,
             cap * hq * 64 * D * 2, blocks * 64 * 64 * 2, blocks * 64 * 4]
    for sz in after:
        off = _align(off + sz)
    return cap, wf, off, _align(off + blocks * 128 * 4)


def _decode_factor(block):
    """[64, 64] from the operand-fragment order: fragment (w, kt), lane
    16 g + c, slot e holds row 16 w + c, column 32 kt + 16 (e / 4) + 4 g + e % 4.
    Fragments (0, 1) and (1, 1) lie above the diagonal and are not stored:
    the workspace handed in is zeroed, so they decode as the zeros they are."""
    out = np.zeros((64, 64))
    b = block.reshape(4, 2, 64, 8)
    for w in range(4):
        for kt in range(2):
            for lane in range(64):
                g, c = lane // 16, lane % 16
                for e in range(8):
                    out[16 * w + c, 32 * kt + 16 * (e // 4) + 4 * g + e % 4] = b[w, kt, lane, e]
    return out


@pytest.mark.parametrize("dtype,l2norm", [("bf16", True), ("f16", False)])
def test_tform_intermediates_match_oracle_chunk_factors(dtype, l2norm):
    # 0539edu section 3.1 (compare intermediates step by step): the stored
    # -T diag(beta) of every chunk and head against oracle.chunk_factors, and
    # the row scales exp(G) / |k|, exp(G_last - G) / |k| (zero past the end)
    from gated_deltanet_chunked_varlen_amd import api, chunk_gated_delta_rule
    from oracle import oracle
    lengths = [130, 1, 64, 200, 65, 90, 17, 128, 40, 77]
    kw = dict(l2norm_in_kernel=True) if l2norm else dict(normalise_in_generator=True)
    wl = W.make(68, lengths, 4, 4, 8, 128, dtype, init="seq", init_std=0.3,
                name="tform_intermediates", **kw)
    assert _tiles_per_cu(wl) > 1
    d = tl.to_device(wl)
    H, D, N, T = wl.H, wl.D, wl.N, wl.T
    cap, wf, gw_end, end = tform_workspace_offsets(T, N, H, D, 4, 4)
    p, _, _ = api.make_params(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"])
    assert api.workspace_size(p) == end
    ws = torch.zeros(end, dtype=torch.uint8, device="cuda")
    chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=wl.scale,
                           cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=l2norm,
                           initial_state=d["initial_state"], workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    prob = oracle.Problem(q=wl.q, k=wl.k, v=wl.v, cu=wl.cu_seqlens.astype(np.int64), g=wl.g,
                          beta=wl.beta, scale=wl.scale, l2norm=l2norm, init_state=None,
                          state_indices=None, ckpt_every=0, ckpt_cu_starts=None)
    table, cc, n = oracle.chunk_table(wl.cu_seqlens, 64)
    worst_t, worst_r = 0.0, 0.0
    for f in range(n):
        i, c = (int(x) for x in table[f])
        t0 = int(wl.cu_seqlens[i]) + 64 * c
        m = min(64, int(wl.cu_seqlens[i + 1]) - t0)
        for h in range(H):
            ch = h * cap + f
            b = raw[wf + ch * 8192: wf + (ch + 1) * 8192].view(np.uint16)
            if dtype == "f16":
                vals = b.view(np.float16).astype(np.float64)
            else:
                vals = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            got = _decode_factor(vals)
            fa = oracle.chunk_factors(prob, h, t0, m)
            want = np.zeros((64, 64))
            want[:m, :m] = -fa["T"] * fa["beta"][None, :]
            e = tl.rel_l2(got, want)
            worst_t = max(worst_t, e)
            assert e < 2e-2, (f, h, e)
            rows = raw[gw_end + ch * 512: gw_end + (ch + 1) * 512].view(np.float32).astype(np.float64)
            G = fa["G"]
            wa = np.zeros(64)
            wb = np.zeros(64)
            wa[:m] = np.exp(G) / fa["knorm"]
            wb[:m] = np.exp(G[-1] - G) / fa["knorm"]
            np.testing.assert_allclose(rows[:64], wa, rtol=1e-4, atol=1e-7)
            np.testing.assert_allclose(rows[64:], wb, rtol=1e-4, atol=1e-7)
            worst_r = max(worst_r, float(np.max(np.abs(rows[:64] - wa) / np.maximum(np.abs(wa), 1e-30))))
    print("tform intermediates", dtype, "worst factor rel-L2 %.3e" % worst_t,
          "worst row rel %.3e" % worst_r, flush=True)
