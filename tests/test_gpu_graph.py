"""Repeated calls captured in a HIP graph (gitcode "FlashInfer GDN Prefill
完全指南", section "约束与注意点": the call makes no host synchronisation, so it
can be captured and replayed).  The library enqueues kernels only (no memset,
no allocation, no device-to-host copy), so a captured call replays with new
input contents in the same buffers.  Each replay is checked bit for bit
against an eager call on the same inputs (every kernel is deterministic),
with eager work and synchronisation between the replays.
"""
import numpy as np
import pytest

from gated_deltanet_chunked_varlen_amd import (chunk_gated_delta_rule,
                                               gated_delta_rule_decode)
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


def _refill(dst, wl):
    src = tl.to_device(wl)
    for name in ("q", "k", "v", "g", "beta", "initial_state"):
        dst[name].copy_(src[name])


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


@pytest.mark.parametrize("lengths", [[130, 20, 300], [64] * 70])
def test_prefill_graph_replays_match_eager(lengths):
    mk = lambda seed: W.make(seed, lengths, 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                             init="seq", init_std=0.3)
    d = tl.to_device(mk(50))
    N, H, D, T = len(lengths), 4, 128, sum(lengths)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    p, _, _ = api.make_params(d["q"], d["k"], d["v"], d["g"], d["beta"],
                              initial_state=d["initial_state"], output_final_state=True,
                              cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                              output=out, output_state=fin)
    ws = torch.empty(api.workspace_size(p), dtype=torch.uint8, device="cuda")

    def call():
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                               initial_state=d["initial_state"], output_final_state=True,
                               cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                               output=out, output_state=fin, status=st, workspace=ws)

    graph = _capture(call)
    for seed in (51, 52, 53):
        _refill(d, mk(seed))
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_fin, got_st = out.clone(), fin.clone(), int(st.item())
        out.zero_()
        fin.zero_()
        call()                                   # eager, same buffers
        torch.cuda.synchronize()
        assert got_st == 0 and int(st.item()) == 0
        assert torch.equal(got_out, out)
        assert torch.equal(got_fin, fin)


def test_decode_graph_loop_matches_eager():
    # a decode loop as a graph: each replay advances an in-place state pool
    N, H, D = 16, 4, 128
    mk = lambda seed: W.make(seed, [1] * N, H, H, H, D, "bf16", l2norm_in_kernel=True,
                             init="pool", pool_size=32, init_std=0.3)
    wl = mk(60)
    d = tl.to_device(wl)
    pool_g = d["initial_state"].clone()
    pool_e = d["initial_state"].clone()
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")

    def step(pool):
        gated_delta_rule_decode(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                initial_state=pool, output_state=pool,
                                state_indices=d["state_indices"],
                                use_qk_l2norm_in_kernel=True, output=out)

    snapshot = pool_g.clone()
    graph = _capture(lambda: step(pool_g))
    pool_g.copy_(snapshot)                        # undo the warm-up step
    for seed in (61, 62, 63, 64):
        new = tl.to_device(mk(seed))
        for name in ("q", "k", "v", "g", "beta"):
            d[name].copy_(new[name])
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step(pool_e)                              # eager on its own pool
        torch.cuda.synchronize()
        assert torch.equal(got, out)
        assert torch.equal(pool_g, pool_e)


def _buffer_set(seed, lengths, H, D, mk):
    d = tl.to_device(mk(seed))
    N, T = len(lengths), sum(lengths)
    d["out"] = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    d["fin"] = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    d["st"] = torch.empty(1, dtype=torch.int32, device="cuda")
    return d


def _args(d):
    return dict(initial_state=d["initial_state"], output_final_state=True,
                cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                output=d["out"], output_state=d["fin"], status=d["st"])


def test_rotating_buffer_sets_replay_bit_equal_to_eager():
    # gitcode "FlashInfer GDN Prefill 完全指南", section "内部机制：plan 缓存、
    # 地址重绑定与 CUDA Graph": three sets of q/k/v/output buffers used in
    # turn (triple buffering); each set is captured once and replayed after,
    # with new contents, eager work and synchronisation between replays
    lengths, H, D = [130, 20, 300, 1, 64], 4, 128
    mk = lambda seed: W.make(seed, lengths, H, H, H, D, "bf16", l2norm_in_kernel=True,
                             init="seq", init_std=0.3)
    sets = [_buffer_set(70 + i, lengths, H, D, mk) for i in range(3)]
    assert len({s["q"].data_ptr() for s in sets}) == 3
    assert len({s["out"].data_ptr() for s in sets}) == 3
    graphs = api.PrefillGraphs()
    seed = 80
    for rnd in range(3):
        for s in sets:
            _refill(s, mk(seed))
            seed += 1
            got_out, got_fin = graphs(s["q"], s["k"], s["v"], s["g"], s["beta"], **_args(s))
            assert got_out.data_ptr() == s["out"].data_ptr()
            torch.cuda.synchronize()
            got_out, got_fin, got_st = got_out.clone(), got_fin.clone(), int(s["st"].item())
            # eager work between replays: an unrelated product and a call
            # into fresh output buffers through the cached workspace
            junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
            e_out, e_fin = chunk_gated_delta_rule(
                s["q"], s["k"], s["v"], s["g"], s["beta"],
                initial_state=s["initial_state"], output_final_state=True,
                cu_seqlens=s["cu_seqlens"], use_qk_l2norm_in_kernel=True)
            torch.cuda.synchronize()
            del junk
            assert got_st == 0
            assert torch.equal(got_out, e_out), (rnd, seed)
            assert torch.equal(got_fin, e_fin), (rnd, seed)
    assert graphs.graphs_captured == 3


def test_workspace_cache_reused_across_rotating_buffers():
    # the plan's workspace is kept per (device, stream): calls whose tensors
    # change address reuse it, a larger call grows it, another stream gets its
    # own, and results match calls given a fresh workspace of their own
    api.clear_workspace_cache()
    lengths, H, D = [300, 64, 17], 4, 128
    mk = lambda seed: W.make(seed, lengths, H, H, H, D, "bf16", l2norm_in_kernel=True,
                             init="seq", init_std=0.3)
    ptrs = set()
    for i in range(3):
        s = tl.to_device(mk(90 + i))
        got = chunk_gated_delta_rule(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                     initial_state=s["initial_state"],
                                     cu_seqlens=s["cu_seqlens"], use_qk_l2norm_in_kernel=True)
        ptrs.add(tuple(w.data_ptr() for w in api._ws_cache.values()))
        p, _, _ = api.make_params(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                  initial_state=s["initial_state"],
                                  cu_seqlens=s["cu_seqlens"], use_qk_l2norm_in_kernel=True)
        ws = torch.zeros(api.workspace_size(p), dtype=torch.uint8, device="cuda")
        ref = chunk_gated_delta_rule(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                     initial_state=s["initial_state"],
                                     cu_seqlens=s["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                                     workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
    assert len(ptrs) == 1 and len(api._ws_cache) == 1
    big = tl.to_device(W.make(95, [4096], H, H, H, D, "bf16", l2norm_in_kernel=True))
    chunk_gated_delta_rule(big["q"], big["k"], big["v"], big["g"], big["beta"],
                           cu_seqlens=big["cu_seqlens"], use_qk_l2norm_in_kernel=True)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        chunk_gated_delta_rule(big["q"], big["k"], big["v"], big["g"], big["beta"],
                               cu_seqlens=big["cu_seqlens"], use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    assert len(api._ws_cache) == 2
    api.clear_workspace_cache()


def test_context_parallel_call_replays_bit_equal_to_eager():
    # the context-parallel form (four kernels, no memset) under capture, with
    # rotated buffer sets: each replay equals an eager call bit for bit
    lengths, H, D = [1000, 333], 2, 128
    mk = lambda seed: W.make(seed, lengths, H, H, H, D, "bf16", l2norm_in_kernel=True,
                             init="seq", init_std=0.3)
    sets = [_buffer_set(130 + i, lengths, H, D, mk) for i in range(2)]
    graphs = api.PrefillGraphs()
    seed = 140
    for rnd in range(2):
        for s in sets:
            _refill(s, mk(seed))
            seed += 1
            got_out, got_fin = graphs(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                      use_cp=True, _cp_chunk_len=256, **_args(s))
            torch.cuda.synchronize()
            got_out, got_fin = got_out.clone(), got_fin.clone()
            e_out, e_fin = chunk_gated_delta_rule(
                s["q"], s["k"], s["v"], s["g"], s["beta"], initial_state=s["initial_state"],
                output_final_state=True, cu_seqlens=s["cu_seqlens"],
                use_qk_l2norm_in_kernel=True, use_cp=True, _cp_chunk_len=256)
            torch.cuda.synchronize()
            assert int(s["st"].item()) == 0
            assert torch.equal(got_out, e_out) and torch.equal(got_fin, e_fin), (rnd, seed)
    assert graphs.graphs_captured == 2


def test_tform_call_replays_bit_equal_to_eager():
    # the T form of the four-tile pass (raw k / v rows loaded by the state
    # pass, no memset) under capture, with rotated buffer sets: each replay
    # equals an eager call bit for bit
    lengths = [300, 1, 64, 129, 250, 90, 200, 77, 140, 33, 180, 65, 100, 150, 210, 40]
    H, D = 8, 128
    mk = lambda seed: W.make(seed, lengths, H, H, H, D, "bf16", l2norm_in_kernel=True,
                             init="seq", init_std=0.3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert len(lengths) * H * (D // 16) >= 4 * cus
    sets = [_buffer_set(150 + i, lengths, H, D, mk) for i in range(2)]
    graphs = api.PrefillGraphs()
    seed = 160
    for rnd in range(2):
        for s in sets:
            _refill(s, mk(seed))
            seed += 1
            got_out, got_fin = graphs(s["q"], s["k"], s["v"], s["g"], s["beta"], **_args(s))
            torch.cuda.synchronize()
            got_out, got_fin = got_out.clone(), got_fin.clone()
            e_out, e_fin = chunk_gated_delta_rule(
                s["q"], s["k"], s["v"], s["g"], s["beta"], initial_state=s["initial_state"],
                output_final_state=True, cu_seqlens=s["cu_seqlens"],
                use_qk_l2norm_in_kernel=True)
            torch.cuda.synchronize()
            assert int(s["st"].item()) == 0
            assert torch.equal(got_out, e_out) and torch.equal(got_fin, e_fin), (rnd, seed)
    assert graphs.graphs_captured == 2
