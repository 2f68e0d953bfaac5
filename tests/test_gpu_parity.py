"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Relative L2 error per tensor: <= 1e-4 for fp32 inputs, <= 2e-2 for bf16
inputs.  The chunk table and pool indexing are compared bit for bit.  The
five named workloads run at their full sizes in the launch configuration the
benchmark times; where the oracle would take too long (the long single
sequence) it is evaluated on sampled heads.
"""
import numpy as np
import pytest

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
    errs, _ = tl.compare(wl, gpu, orc, heads)
    bars = tl.bars(wl)
    print(wl.name, {k: "%.3e" % v for k, v in errs.items()}, "bars", bars, flush=True)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])
    return errs


# --------------------------------------------------------------- chunk table

CU_CASES = [
    [0, 130, 150, 450],                      # the weigao.cc example
    [0, 130, 150, 450, 450, 514, 515],       # ragged with an empty sequence
    [0, 0, 0],                               # all empty
    [0],                                     # no sequences
    [0, 64, 128, 192],                       # exact multiples
    [0, 1],                                  # a single token
    [0, 262144],                             # one long sequence
]


@pytest.mark.parametrize("cu", CU_CASES + ["random_big"])
@pytest.mark.parametrize("itype", ["int32", "int64"])
def test_chunk_index_bitexact(cu, itype):
    from gated_deltanet_chunked_varlen_amd import build_chunk_indices
    if cu == "random_big":
        rng = np.random.default_rng(5)
        lens = rng.integers(0, 200, 2500)
        lens[rng.random(2500) < 0.2] = 0
        cu = np.concatenate([[0], np.cumsum(lens)])
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    dev = torch.from_numpy(cu.astype(itype)).cuda()
    table, cc, starts, n, st = build_chunk_indices(dev, T)
    torch.cuda.synchronize()
    want_t, want_cc, want_n = oracle.chunk_table(cu, 64)
    assert int(n.item()) == want_n
    assert int(st.item()) == 0
    np.testing.assert_array_equal(cc.cpu().numpy(), want_cc)
    np.testing.assert_array_equal(starts.cpu().numpy(), cu.astype(np.int32))
    got = table.cpu().numpy()
    np.testing.assert_array_equal(got[:want_n], want_t)
    assert (got[want_n:] == -1).all()


def test_chunk_index_flags_bad_cu_seqlens():
    from gated_deltanet_chunked_varlen_amd import build_chunk_indices
    cu = torch.tensor([0, 100, 50, 300, 200], dtype=torch.int32, device="cuda")
    table, cc, starts, n, st = build_chunk_indices(cu, 250)
    torch.cuda.synchronize()
    assert int(st.item()) & 1
    s = starts.cpu().numpy()
    assert (np.diff(s) >= 0).all() and s[-1] <= 250 and s[0] == 0
    assert int(n.item()) <= table.shape[0]


# ------------------------------------------------------------- named configs

def test_single_l128_h1_d32_f32_fp32():
    wl = W.single_l128_h1_d32_f32()
    gpu = tl.run_gpu(wl)
    orc = tl.run_oracle(wl)
    _check(wl, gpu, orc)
    # elementwise, the tolerance 0539edu section 3.4 suggests
    np.testing.assert_allclose(gpu["out"], orc["out"], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(gpu["final"], orc["final"], rtol=1e-4, atol=1e-5)


def test_varlen_2x2048_h16_d128():
    wl = W.varlen_2x2048_h16_d128()
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


def test_ragged6_pool64_h16_d128_in_place():
    wl = W.ragged6_pool64_h16_d128()
    gpu = tl.run_gpu(wl, status=True)
    orc = tl.run_oracle(wl)
    assert gpu["status"] == 0
    _check(wl, gpu, orc)
    # rows not addressed by state_indices are bitwise unchanged
    idx = set(int(r) for r in wl.state_indices)
    others = [r for r in range(wl.initial_state.shape[0]) if r not in idx]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])
    # the empty sequence keeps its state exactly
    empty = int(wl.state_indices[3])
    np.testing.assert_array_equal(gpu["final"][empty], gpu["pool_before"][empty])


# ---------------------------------------------------------------- edge cases

def _small(seed, lengths, dtype="bf16", hq=2, hk=2, hv=2, D=128, **kw):
    kw.setdefault("l2norm_in_kernel", True)
    return W.make(seed, lengths, hq, hk, hv, D, dtype, **kw)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("bf16", 32),
                                     ("f16", 128), ("f16", 64), ("f16", 32),
                                     ("f32", 128), ("f32", 64), ("f32", 32)])
def test_dtype_and_head_size(dtype, D):
    wl = _small(11, [200, 64, 0, 65, 3], dtype=dtype, D=D, init="seq")
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


@pytest.mark.parametrize("hq,hk,hv", [(4, 2, 2), (2, 2, 6), (3, 3, 3)])
def test_head_sharing(hq, hk, hv):
    wl = _small(12, [100, 70], hq=hq, hk=hk, hv=hv)
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


def test_defaults_no_gates_no_scale():
    wl = _small(13, [150, 40], gates=False, qkv_std=1.0)
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


def test_explicit_scale_and_no_l2norm():
    wl = _small(14, [90], normalise_in_generator=True, l2norm_in_kernel=False,
                scale=0.3)
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


def test_empty_batch_and_zero_lengths():
    wl = _small(15, [0, 0, 0], init="seq")
    gpu = tl.run_gpu(wl)
    # no tokens: final state = initial state, converted to fp32
    np.testing.assert_array_equal(gpu["final"], wl.initial_state.astype(np.float64))


def test_int64_metadata_and_pool_not_in_place():
    wl = _small(16, [33, 130, 7], init="pool", pool_size=9,
                cu_dtype=np.int64)
    wl.state_indices = wl.state_indices.astype(np.int64)
    gpu = tl.run_gpu(wl)
    orc = tl.run_oracle(wl)
    _check(wl, gpu, orc)


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
def test_state_dtypes(sdt):
    wl = _small(17, [300, 20], init="seq", init_dtype="bf16")
    wl.final_state_dtype = sdt
    gpu = tl.run_gpu(wl)
    orc = tl.run_oracle(wl)
    _check(wl, gpu, orc)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_pool_in_place_and_fp8_checkpoints(fmt):
    """8-bit float states (gitcode, section "chunk_gated_delta_rule API
    全参数解析" lists fp8 initial states, section "中间状态检查点" fp8
    checkpoints): the pool is read and written in place in ``fmt`` and the
    checkpoints are stored in ``fmt``.  The pool rows the call does not touch
    keep their bits."""
    wl = _small(21, [200, 64, 0, 131], init="pool", pool_size=9, in_place_pool=True,
                init_dtype=fmt, final_state_dtype=fmt, checkpoint_every=64,
                checkpoint_dtype=fmt, init_std=0.3)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    idx = set(int(r) for r in wl.state_indices)
    others = [r for r in range(9) if r not in idx]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_final_state_rounds_like_torch(fmt):
    """The fp8 store is round to nearest, ties to even: the fp8 final state
    of a call equals, bit for bit, torch's conversion of the fp32 final state
    of the same call (values far inside the format's range)."""
    wl = _small(22, [150, 70], init="seq", init_std=0.3)
    ref = tl.run_gpu(wl)["final"]
    wl8 = _small(22, [150, 70], init="seq", init_std=0.3, final_state_dtype=fmt)
    got = tl.run_gpu(wl8)["final"]
    dt = tl.state_torch_dtype(fmt)
    want = torch.from_numpy(ref.astype(np.float32)).to(dt).to(torch.float32).numpy()
    assert np.abs(ref).max() < 100.0
    np.testing.assert_array_equal(got, want.astype(np.float64))


def test_strided_states():
    """Initial and final states as non-contiguous views ([v][k] order kept,
    heads and rows interleaved differently)."""
    wl = _small(18, [140, 64], init="seq")
    H, D, N = wl.H, wl.D, wl.N
    base = torch.from_numpy(np.ascontiguousarray(
        wl.initial_state.transpose(1, 0, 2, 3))).cuda()       # [H, N, V, K]
    init = base.permute(1, 0, 2, 3)                            # [N, H, V, K] view
    outbuf = torch.zeros((H, D, D, N), dtype=torch.float32, device="cuda")
    outst = outbuf.permute(3, 0, 1, 2)                         # [N, H, V, K] view
    gpu = tl.run_gpu(wl, initial_state=init, output_state=outst)
    orc = tl.run_oracle(wl)
    _check(wl, dict(gpu, final=outst.cpu().numpy().astype(np.float64)), orc)


def test_checkpoints_every_64_and_bf16_checkpoint_rows():
    wl = _small(19, [300, 64, 130, 0], init="seq", checkpoint_every=64)
    _check(wl, tl.run_gpu(wl), tl.run_oracle(wl))


def test_determinism_bitwise():
    wl = W.ragged6_pool64_h16_d128()
    a = tl.run_gpu(wl)
    b = tl.run_gpu(wl)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["final"], b["final"])


def test_continuation_split_runs():
    """Running a sequence in two calls, passing the first call's final state
    as the second's initial state, matches one call (weigao.cc, section
    "chunked prefill 有两层含义": scheduler-level chunked prefill)."""
    wl = _small(20, [500], init="seq")
    full = tl.run_gpu(wl)
    cut = 130
    a = W.make(20, [500], 2, 2, 2, 128, "bf16", l2norm_in_kernel=True, init="seq")
    first = W.Workload(**{**a.__dict__})
    first.q, first.k, first.v = a.q[:cut], a.k[:cut], a.v[:cut]
    first.g, first.beta = a.g[:cut], a.beta[:cut]
    first.cu_seqlens = np.array([0, cut], dtype=np.int32)
    r1 = tl.run_gpu(first)
    second = W.Workload(**{**a.__dict__})
    second.q, second.k, second.v = a.q[cut:], a.k[cut:], a.v[cut:]
    second.g, second.beta = a.g[cut:], a.beta[cut:]
    second.cu_seqlens = np.array([0, 500 - cut], dtype=np.int32)
    second.initial_state = r1["final"].astype(np.float32)
    r2 = tl.run_gpu(second)
    out = np.concatenate([r1["out"], r2["out"]])
    assert tl.rel_l2(out, full["out"]) < 2e-2
    assert tl.rel_l2(r2["final"], full["final"]) < 2e-2


# ------------------------------------------------------- device status words

def test_status_bad_state_index_writes_nothing():
    wl = _small(21, [70, 40], init="pool", pool_size=4, in_place_pool=True)
    wl.state_indices = np.array([1, 9], dtype=np.int32)    # 9 is out of range
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] & 4
    for r in (0, 2, 3):
        np.testing.assert_array_equal(gpu["final"][r], gpu["pool_before"][r])


def test_status_checkpoint_starts_mismatch():
    wl = _small(22, [300, 130], init="seq", checkpoint_every=64)
    wl.checkpoint_cu_starts = wl.checkpoint_cu_starts.copy()
    wl.checkpoint_cu_starts[1] += 1                         # inconsistent
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] & 2


def test_f16_two_by_2048_pool_f16_states():
    # fp16 inputs with fp16 pool states at the 2 x 2048, 16-head shape
    wl = W.make(33, [2048, 2048], 16, 16, 16, 128, "f16", l2norm_in_kernel=True,
                init="pool", pool_size=4, init_dtype="f16", in_place_pool=True)
    wl.initial_state_dtype = "f16"
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_many_sequences_chunk_table_path():
    # more sequences than one wave holds: the chunk-index builder's tables
    # drive every kernel (fewer use the geometry straight from cu_seqlens)
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(0, 150, size=100)]
    lengths[5] = lengths[40] = 0
    wl = _small(31, lengths, D=64, init="pool", pool_size=128, checkpoint_every=64)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_sequences_than_one_scan_block(dtype):
    # 1500 sequences: the chunk-index builder's scan takes several passes of
    # its block, inside a whole call, with a pool of 1600 rows in place
    rng = np.random.default_rng(33)
    lengths = [int(x) for x in rng.integers(0, 90, size=1500)]
    for i in rng.choice(1500, 200, replace=False):
        lengths[int(i)] = 0
    wl = _small(33, lengths, dtype=dtype, D=32, init="pool", pool_size=1600,
                in_place_pool=True, checkpoint_every=64)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))
    rows = set(int(r) for r in wl.state_indices)
    others = [r for r in range(1600) if r not in rows]
    np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])


# Batches whose one-tile state-pass grid outgrows the CUs take two 16-column
# tiles per workgroup and start the longest sequences first.  Configs 3 and 4
# and the chunk-table case above reach that only at D = 128 or through the
# table; these reach it in the direct (up to 63 sequences) geometry at every
# head size, with uneven lengths, an empty sequence, pools and checkpoints.
TWO_TILE_CASES = {
    "d64_f16_pool": dict(heads=(12, 12, 12), D=64, dtype="f16", l2norm_in_kernel=True,
                         init="pool", pool_size=48, in_place_pool=True, init_dtype="f16",
                         final_state_dtype="f16", checkpoint_every=128),
    "d32_bf16_gqa": dict(heads=(16, 4, 4), D=32, dtype="bf16", normalise_in_generator=True,
                         init="seq", init_dtype="bf16", checkpoint_every=64),
    "d128_bf16_gva_e4m3": dict(heads=(4, 4, 8), D=128, dtype="bf16", l2norm_in_kernel=True,
                               init="pool", pool_size=41, in_place_pool=True,
                               init_dtype="e4m3", final_state_dtype="e4m3"),
}


@pytest.mark.parametrize("case", sorted(TWO_TILE_CASES))
def test_two_tile_workgroups(case):
    kw = dict(TWO_TILE_CASES[case])
    hq, hk, hv = kw.pop("heads")
    D, dtype = kw.pop("D"), kw.pop("dtype")
    seed = 40 + sorted(TWO_TILE_CASES).index(case)
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, 400, size=40)]
    lengths[7] = 0
    wl = W.make(seed, lengths, hq, hk, hv, D, dtype, name="two_tile_" + case, **kw)
    assert wl.N * wl.H * (D // 16) > 256, "the case must outgrow one round of workgroups"
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


def test_sequence_results_do_not_depend_on_batch_position():
    # Every (sequence, head, tile) is computed on its own: taking the batch in
    # another order (here reversed, 40 uneven sequences, so the state pass
    # takes two tiles per workgroup and starts the longest sequences first)
    # must give each sequence bit-identical outputs and final states.
    import copy
    rng = np.random.default_rng(45)
    lengths = [int(x) for x in rng.integers(1, 400, size=40)]
    lengths[11] = 0
    a = W.make(45, lengths, 8, 8, 8, 128, "bf16", l2norm_in_kernel=True, init="seq",
               name="order_a")
    assert a.N * a.H * 8 > 256
    cu = a.cu_seqlens.astype(np.int64)
    order = list(range(a.N))[::-1]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order]).astype(np.int64)
    b = copy.deepcopy(a)
    b.q, b.k, b.v = a.q[rows], a.k[rows], a.v[rows]
    b.g, b.beta = a.g[rows], a.beta[rows]
    b.initial_state = a.initial_state[order]
    nl = [lengths[i] for i in order]
    b.cu_seqlens = np.concatenate([[0], np.cumsum(nl)]).astype(a.cu_seqlens.dtype)
    ra, rb = tl.run_gpu(a), tl.run_gpu(b)
    cub = b.cu_seqlens.astype(np.int64)
    for pos, i in enumerate(order):
        assert np.array_equal(ra["out"][cu[i]:cu[i + 1]], rb["out"][cub[pos]:cub[pos + 1]]), i
        assert np.array_equal(ra["final"][i], rb["final"][pos]), i


@pytest.mark.parametrize("nseq", [3, 80])
def test_status_bad_cu_seqlens_full_call(nseq):
    # a decreasing offset is flagged on both geometry paths (up to 63
    # sequences the kernels check it themselves, beyond that the builder
    # does), and the call still completes
    lengths = [40] * nseq
    wl = _small(32, lengths)
    cu = wl.cu_seqlens.copy()
    cu[2] = cu[1] - 5
    wl.cu_seqlens = cu
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] & 1
    assert np.isfinite(gpu["out"]).all()


def test_host_errors_raise_before_launch():
    from gated_deltanet_chunked_varlen_amd import chunk_gated_delta_rule
    wl = _small(23, [64, 64])
    d = tl.to_device(wl)
    with pytest.raises(ValueError):
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"],
                               checkpoint_every_n_tokens=100,
                               state_checkpoints=torch.zeros(4, 2, 128, 128, device="cuda"),
                               checkpoint_cu_starts=torch.zeros(3, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"],
                               max_seqlen=10)
    with pytest.raises(ValueError):
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], cu_seqlens=d["cu_seqlens"],
                               output_final_state=True,
                               state_indices=torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
                               initial_state=torch.zeros(4, 2, 128, 128, device="cuda"))


# ------------------------------------------------- large named configs (last)

def test_gva8_h16x32_d128_checkpoints():
    wl = W.gva8_h16x32_d128_checkpoints()
    heads = [0, 1, 17, 31]
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    orc = tl.run_oracle(wl, heads=heads)
    _check(wl, gpu, orc, heads=heads)


# Calls whose intermediates outgrow the last-level cache (above 200 MiB,
# counted over the chunk-count bound the workspace uses) take the large-call
# form: non-temporal intermediate stores and the L2 warm-up wave of the state
# pass.  The configs above reach it only at D = 128; these two reach it at
# D = 64 (fp16, in-kernel norm, in-place pool, checkpoints) and at D = 32
# (bf16, no norm, GQA), checked on every head.
LARGE_CALL_BYTES = 200 << 20


def _assert_large_call(wl):
    chunks = (wl.T + 63 * wl.N) // 64
    inter = chunks * wl.H * (4 * 64 * wl.D + 64 * 64) * 2
    assert inter > LARGE_CALL_BYTES, inter


@pytest.mark.timeout(600)
def test_large_call_form_d64_f16_pool_checkpoints():
    wl = W.make(31, [8000, 6500, 7200], 16, 16, 16, 64, "f16", l2norm_in_kernel=True,
                init="pool", pool_size=7, in_place_pool=True, checkpoint_every=1024,
                name="large_d64_f16")
    _assert_large_call(wl)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


@pytest.mark.timeout(600)
def test_large_call_form_d32_bf16_gqa():
    wl = W.make(32, [9800, 130, 8000], 32, 8, 8, 32, "bf16", normalise_in_generator=True,
                init="seq", name="large_d32_bf16")
    _assert_large_call(wl)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    _check(wl, gpu, tl.run_oracle(wl))


@pytest.mark.timeout(600)
def test_long_l262144_h32_d128_sampled_heads():
    wl = W.long_l262144_h32_d128()
    heads = [0, 9, 22, 31]
    gpu = tl.run_gpu(wl)
    orc = tl.run_oracle(wl, heads=heads)
    _check(wl, gpu, orc, heads=heads)
