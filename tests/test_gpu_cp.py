"""GPU parity of the context-parallel prefill (use_cp) against the oracle,
through the C ABI.

Context parallelism cuts each sequence into segments, forms every segment's
transition pair at once, fixes the segment start states up serially and runs
every segment from its start (gitcode "FlashInfer GDN Prefill 完全指南",
section "Cake GDN CP 后端", "四阶段执行流程"; 0539edu "GDN与线性注意力GPU并行
实现", sections 2.1-2.2: the per-chunk update is affine in the state and such
maps compose).  It computes the same recurrence in another order, so the
oracle's token recurrence is still its definition and the bars are those of
the ordinary pass; the block maxima localise an error to one 64-token chunk
and head, hence to one segment.  Segment lengths are forced small
(_cp_chunk_len) so that short sequences cross several segment boundaries,
including boundaries that fall inside a checkpoint interval and sequences
shorter than one segment.
"""
import numpy as np
import pytest

from gated_deltanet_chunked_varlen_amd import api, chunk_gated_delta_rule
from gated_deltanet_chunked_varlen_amd import _native as nat
from gated_deltanet_chunked_varlen_amd import workloads as W
from oracle import oracle
from tests import gdn_testlib as tl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _check(wl, gpu, orc, heads=None):
    errs, _ = tl.compare(wl, gpu, orc, heads=heads)
    bars = tl.bars(wl)
    print(wl.name, {k: "%.3e" % v for k, v in errs.items()}, "bars", bars, flush=True)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])


@pytest.mark.parametrize("dtype,seg", [("bf16", 256), ("bf16", 64), ("f16", 192)])
def test_cp_single_sequence_segments(dtype, seg):
    wl = W.make(120, [1000], 2, 2, 2, 128, dtype, l2norm_in_kernel=True, init="seq",
                init_std=0.3, checkpoint_every=128)
    gpu = tl.run_gpu(wl, status=True, use_cp=True, _cp_chunk_len=seg)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_cp_varlen_gva_in_place_pool():
    # zero-length and one-token sequences, a sequence shorter than one
    # segment, GVA heads, an in-place pool addressed by state_indices
    wl = W.make(121, [300, 0, 700, 64, 1, 129], 2, 2, 4, 128, "bf16", l2norm_in_kernel=True,
                init="pool", pool_size=9, in_place_pool=True, init_std=0.3)
    gpu = tl.run_gpu(wl, status=True, use_cp=True, _cp_chunk_len=128)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    idx = set(int(r) for r in wl.state_indices)
    others = [r for r in range(9) if r not in idx]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


def test_cp_gqa_checkpoints_bf16_states():
    wl = W.make(122, [1500, 640], 4, 2, 2, 128, "bf16", l2norm_in_kernel=True, init="seq",
                init_std=0.3, checkpoint_every=256, final_state_dtype="bf16",
                checkpoint_dtype="bf16")
    gpu = tl.run_gpu(wl, status=True, use_cp=True, _cp_chunk_len=320)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_cp_auto_takes_long_few_head_calls_and_matches():
    # one 16 384-token sequence with two heads fills 16 of the 256 compute
    # units; "auto" takes the context-parallel pass (more workspace than the
    # ordinary pass) and matches the oracle
    wl = W.make(123, [16384], 2, 2, 2, 128, "bf16", l2norm_in_kernel=True, init="seq",
                init_std=0.3)
    d = tl.to_device(wl)
    sizes = {}
    for mode in ("auto", False):
        p, _, _ = api.make_params(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"],
                                  use_cp=mode)
        sizes[mode] = api.workspace_size(p)
    assert sizes["auto"] > sizes[False]
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_cp_matches_the_ordinary_pass_closely():
    # the two passes round differently (the segment transitions are formed in
    # bf16 operands like the chain itself), so they agree to rounding
    wl = W.make(124, [2048, 777], 4, 4, 4, 128, "bf16", l2norm_in_kernel=True, init="seq",
                init_std=0.3)
    a = tl.run_gpu(wl, use_cp=True, _cp_chunk_len=512)
    b = tl.run_gpu(wl, use_cp=False)
    assert tl.rel_l2(a["out"], b["out"]) < 1e-2
    assert tl.rel_l2(a["final"], b["final"]) < 1e-2


def test_cp_on_outside_its_domain_fails_closed():
    wl = W.make(125, [256], 2, 2, 2, 64, "bf16")
    d = tl.to_device(wl)
    with pytest.raises(Exception) as e:
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"], use_cp=True)
    assert "GDN_ERR_CP" in str(e.value) or "use_cp" in str(e.value)


@pytest.mark.timeout(900)
def test_cp_long_l262144_h32_d128_sampled_heads():
    # the 262 144-token, 32-head call in eight segments of 32 768 tokens
    wl = W.long_l262144_h32_d128()
    heads = [0, 13, 31]
    gpu = tl.run_gpu(wl, use_cp=True, _cp_chunk_len=32768)
    orc = tl.run_oracle(wl, heads=heads)
    _check(wl, gpu, orc, heads=heads)


def test_cp_auto_long_l65536_h4_bench_workload():
    # the workload the bench times with and without context parallelism
    wl = W.long_l65536_h4_d128()
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def _align(x):
    return (x + 255) // 256 * 256


def cp_workspace_offsets(T, N, H, D, nseg, hq=None, hk=None):
    """Byte offsets of the context-parallel buffers in a 16-bit call's
    workspace (the layout of gdn_prefill_workspace_size: chunk tables, then
    W, the k fragments (per k head), U, the q fragments (per q head), P,
    gates, the T form's row scales, then the segment start states, local
    states and transitions, each 256-byte aligned)."""
    cap = int(nat.lib().gdn_max_chunks(T, N))
    blocks = cap * H
    kb, qb = cap * (hk or H), cap * (hq or H)
    sizes = [8 * max(cap, 1), 8 * max(cap, 1), 4 * (N + 1), 4 * (N + 1), 4,
             blocks * 64 * D * 2, kb * 64 * D * 2, blocks * 64 * D * 2,
             qb * 64 * D * 2, blocks * 64 * 64 * 2, blocks * 64 * 4, blocks * 128 * 4]
    off = 0
    for sz in sizes:
        off = _align(off + sz)
    st = N * nseg * H * D * D * 4
    start = off
    sloc = _align(start + st)
    mt = _align(sloc + st)
    return start, sloc, mt, _align(mt + st)


def _decode_m(block, D):
    """The transition M[k][m] from its stored operand order."""
    k = np.arange(D)[:, None]
    m = np.arange(D)[None, :]
    idx = (((k // 16) * (D // 16) + m // 16) * 64 + 16 * (m % 4) + k % 16) * 4 + (m // 4) % 4
    return block[idx]


def test_cp_segment_pairs_and_start_states_match_oracle():
    # gitcode, "四阶段执行流程" (M/N precompute, state fix-up) and 0539edu
    # section 2.1 (a run of chunks acts on its start state as an affine map):
    # each non-final segment's local state is the segment run from zero,
    # its transition M satisfies run(X) - run(0) = M X for any start X, and
    # each segment start state is the prefix run from the initial state
    lengths, H, D, seg = [1000, 300], 2, 128, 256
    wl = W.make(126, lengths, H, H, H, D, "bf16", l2norm_in_kernel=True, init="seq",
                init_std=0.3)
    d = tl.to_device(wl)
    N, T = wl.N, wl.T
    nseg = -(-(-(-T // 64)) // (seg // 64))
    start_off, sloc_off, m_off, end = cp_workspace_offsets(T, N, H, D, nseg)
    p, _, _ = api.make_params(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"],
                              use_cp=True, _cp_chunk_len=seg)
    assert api.workspace_size(p) == end
    ws = torch.zeros(end, dtype=torch.uint8, device="cuda")
    chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=wl.scale,
                           cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                           initial_state=d["initial_state"], output_final_state=True,
                           use_cp=True, _cp_chunk_len=seg, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    blk = D * D * 4
    f32 = lambda off, i, p_, h: raw[off + (((i * nseg + p_) * H + h) * blk):
                                    off + (((i * nseg + p_) * H + h) * blk) + blk].view(np.float32)
    rng = np.random.default_rng(7)
    cu = wl.cu_seqlens.astype(np.int64)

    def run(b, e, init):
        prob = oracle.Problem(q=wl.q[b:e], k=wl.k[b:e], v=wl.v[b:e], cu=np.array([0, e - b]),
                              g=wl.g[b:e], beta=wl.beta[b:e], scale=wl.scale, l2norm=True,
                              init_state=init, state_indices=None, ckpt_every=0,
                              ckpt_cu_starts=None)
        return oracle.token(prob)["final"][0]            # [H, V, K]

    checked = 0
    for i in range(N):
        b, e = int(cu[i]), int(cu[i + 1])
        used = max(1, -(-(e - b) // seg))
        for p_ in range(used):
            sb = b + seg * p_
            want_start = run(b, sb, wl.initial_state[i:i + 1]) if p_ > 0 else wl.initial_state[i]
            got_start = np.stack([f32(start_off, i, p_, h).reshape(D, D) for h in range(H)])
            assert tl.rel_l2(got_start, want_start) < 2e-2, (i, p_)
            if p_ + 1 >= used:
                continue
            se = sb + seg
            zero = run(sb, se, None)
            got_loc = np.stack([f32(sloc_off, i, p_, h).reshape(D, D) for h in range(H)])
            assert tl.rel_l2(got_loc, zero) < 2e-2, (i, p_)
            X = rng.standard_normal((1, H, D, D)) * 0.3
            delta = run(sb, se, X) - zero                    # [H, V, K] = X_h M_h^T
            for h in range(H):
                M = _decode_m(f32(m_off, i, p_, h), D)
                assert tl.rel_l2(X[0, h] @ M.T, delta[h]) < 2e-2, (i, p_, h)
            checked += 1
    assert checked >= 3
