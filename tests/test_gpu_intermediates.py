"""GPU checks below the call's outputs (0539edu "GDN与线性注意力GPU并行实现",
section 3.1: compare step by step against a reference).

* fp32 inputs keep the chunk-start states and the new values N in the
  workspace; they are decoded and compared with the oracle's chunked-form
  dump (``oracle.chunked(..., dump=True)``), chunk by chunk and head by head.
* States stored narrower than fp32 (bf16, fp16, fp8 E4M3 / E5M2) must equal,
  bit for bit, the same call's fp32 states rounded by torch (round to
  nearest even).  Together with the fp32 states' own parity against the
  oracle this pins both the computation and the placement of every final,
  pool and checkpoint row.
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


def _align(x):
    return (x + 255) // 256 * 256


def fp32_workspace_offsets(T, N, H, D):
    """Byte offsets of N and the chunk-start states in the fp32 workspace
    (the layout of gdn_prefill_workspace_size: chunk tables, then W, Ktilde,
    U, N, chunk-start states, gates, each 256-byte aligned)."""
    from gated_deltanet_chunked_varlen_amd import _native
    cap = int(_native.lib().gdn_max_chunks(T, N))
    blocks = cap * H
    off = 0
    sizes = [8 * max(cap, 1), 8 * max(cap, 1), 4 * (N + 1), 4 * (N + 1), 4,
             blocks * 64 * D * 4, blocks * 64 * D * 4, blocks * 64 * D * 4]
    for sz in sizes:
        off = _align(off + sz)
    nf = off
    hf = _align(nf + blocks * 64 * D * 4)
    return cap, nf, hf


def pi(g, s):
    return 16 * (s // 4) + 4 * g + (s % 4)


@pytest.mark.parametrize("D", [32, 64])
def test_fp32_chunk_states_and_new_values_match_oracle_dump(D):
    from gated_deltanet_chunked_varlen_amd import chunk_gated_delta_rule
    lengths = [200, 64, 0, 131]
    wl = W.make(51, lengths, 2, 2, 2, D, "f32", l2norm_in_kernel=True, init="seq",
                name="intermediates_d%d" % D)
    d = tl.to_device(wl)
    H, N, T = wl.H, wl.N, wl.T
    cap, nf_off, hf_off = fp32_workspace_offsets(T, N, H, D)
    ws = torch.zeros(_align(hf_off + cap * H * D * D * 4) + (1 << 20), dtype=torch.uint8,
                     device="cuda")
    chunk_gated_delta_rule(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], scale=wl.scale,
                           cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
                           initial_state=d["initial_state"], output_final_state=True,
                           workspace=ws)
    torch.cuda.synchronize()
    wsf = ws.cpu().numpy()
    orc = oracle.chunked(tl.oracle_problem(wl), 64, dump=True)
    table, cc, n = oracle.chunk_table(wl.cu_seqlens, 64)
    cu = np.asarray(wl.cu_seqlens, np.int64)
    g_of = np.repeat(np.arange(4), 16)
    c_of = np.tile(np.arange(16), 4)
    for f in range(n):
        i, c = (int(x) for x in table[f])
        t0 = int(cu[i]) + 64 * c
        rows = min(64, int(cu[i + 1]) - t0)
        for h in range(H):
            ch = h * cap + f
            # chunk-start state: [D/16 tiles][D/4 slots][64 lanes]
            hb = np.frombuffer(wsf[hf_off + ch * D * D * 4: hf_off + (ch + 1) * D * D * 4].tobytes(),
                               np.float32).reshape(D // 16, D // 4, 64)
            S = np.zeros((D, D))
            for jv in range(D // 16):
                for kt in range(D // 4):
                    S[pi(g_of, kt), 16 * jv + c_of] = hb[jv, kt]
            want = orc["chunk_states"][f, h].T          # stored [v][k] -> S[k][v]
            assert tl.rel_l2(S, want) < 1e-4, (f, h, tl.rel_l2(S, want))
            # new values: [D/16 tiles][16 slots][64 lanes]; rows past the end are 0
            nb = np.frombuffer(wsf[nf_off + ch * 64 * D * 4: nf_off + (ch + 1) * 64 * D * 4].tobytes(),
                               np.float32).reshape(D // 16, 16, 64)
            Nm = np.zeros((64, D))
            for jv in range(D // 16):
                for kt in range(16):
                    Nm[pi(g_of, kt), 16 * jv + c_of] = nb[jv, kt]
            want_n = orc["vnew"][t0:t0 + rows, h]
            assert tl.rel_l2(Nm[:rows], want_n) < 1e-4, (f, h, tl.rel_l2(Nm[:rows], want_n))
            assert np.all(Nm[rows:] == 0.0)


NARROW = ["bf16", "f16", "e4m3", "e5m2"]


@pytest.mark.parametrize("fmt", NARROW)
def test_narrow_final_and_checkpoint_states_are_the_rounded_fp32_states(fmt):
    # the same call with fp32 and with narrow final / checkpoint states: every
    # narrow element equals torch's rounding of the fp32 element; the fp32
    # states themselves are held to the compute bar against the oracle
    base = dict(l2norm_in_kernel=True, init="seq", init_std=0.3, checkpoint_every=64)
    lengths = [300, 64, 0, 131, 65]
    w32 = W.make(52, lengths, 4, 4, 4, 128, "bf16", name="narrow_ref", **base)
    wn = W.make(52, lengths, 4, 4, 4, 128, "bf16", name="narrow_" + fmt,
                final_state_dtype=fmt, checkpoint_dtype=fmt, **base)
    r32, rn = tl.run_gpu(w32), tl.run_gpu(wn)
    errs, _ = tl.compare(w32, r32, tl.run_oracle(w32))
    bars = tl.bars(w32)
    assert all(e <= bars[k] for k, e in errs.items()), errs
    dt = tl.state_torch_dtype(fmt)
    for key in ("final", "ckpt"):
        want = torch.from_numpy(r32[key].astype(np.float32)).to(dt).to(torch.float32).numpy()
        np.testing.assert_array_equal(rn[key], want.astype(np.float64), err_msg=key)
    np.testing.assert_array_equal(rn["out"], r32["out"])


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_narrow_in_place_pool_rows_are_the_rounded_fp32_rows(fmt):
    # a pool read and written in place in `fmt`: the rows the call owns equal
    # the rounding of the same call's fp32 final states (the initial pool
    # holds the same `fmt` values in both calls), every other row keeps its
    # bits
    kw = dict(l2norm_in_kernel=True, init="pool", pool_size=11, init_std=0.3,
              init_dtype=fmt, in_place_pool=True)
    lengths = [200, 64, 0, 131]
    wn = W.make(53, lengths, 2, 2, 2, 128, "bf16", final_state_dtype=fmt, name="pool_" + fmt, **kw)
    rn = tl.run_gpu(wn, status=True)
    assert rn["status"] == 0
    w32 = W.make(53, lengths, 2, 2, 2, 128, "bf16", final_state_dtype="f32", name="pool_ref",
                 **{**kw, "in_place_pool": False})
    # the same initial pool, final states into a separate fp32 pool
    r32 = tl.run_gpu(w32, output_state=torch.zeros((11, w32.H, 128, 128), dtype=torch.float32,
                                                    device="cuda"))
    idx = [int(r) for r in wn.state_indices]
    dt = tl.state_torch_dtype(fmt)
    want = torch.from_numpy(r32["final"][idx].astype(np.float32)).to(dt).to(torch.float32).numpy()
    np.testing.assert_array_equal(rn["final"][idx], want.astype(np.float64))
    others = [r for r in range(11) if r not in set(idx)]
    np.testing.assert_array_equal(rn["final"][others], rn["pool_before"][others])
