"""The calls only enqueue work on the caller's stream and return without
waiting for the device: no host synchronisation and no blocking
device-to-host copy (gitcode "FlashInfer GDN Prefill 完全指南", section
"约束与注意点": the chunk geometry is not read back to the host, so nothing
stalls the host between calls).  A bounded spin kernel is queued ahead of
each call; the stream must still be busy when the call has returned, and
the results must equal those of an earlier call on the same inputs.
"""
import time

import pytest

from gated_deltanet_chunked_varlen_amd import (chunk_gated_delta_rule,
                                               gated_delta_rule_decode)
from gated_deltanet_chunked_varlen_amd import api
from gated_deltanet_chunked_varlen_amd import workloads as W
from tests import gdn_testlib as tl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SPIN_CYCLES = 50_000_000     # a bounded spin (well under a second at any clock)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _returns_while_busy(call):
    """Queue the spin, run call(), report whether the stream was still busy
    when call() returned, and how long call() took on the host."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    t0 = time.perf_counter()
    call()
    dt = time.perf_counter() - t0
    busy = not stream.query()
    torch.cuda.synchronize()
    return busy, dt


# 3 sequences: geometry derived in the kernels; 70 sequences: the
# chunk-index builder runs first and fills the chunk table on the device
@pytest.mark.parametrize("lengths", [[130, 20, 300], [64] * 40 + [1, 65, 127] * 10])
def test_prefill_returns_before_the_device_finishes(lengths):
    wl = W.make(70, lengths, 4, 4, 4, 128, "bf16", l2norm_in_kernel=True,
                init="seq", init_std=0.3, checkpoint_every=64)
    d = tl.to_device(wl)
    N, H, D, T = len(lengths), 4, 128, sum(lengths)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    ck = torch.empty((int(wl.checkpoint_cu_starts[-1]), H, D, D), dtype=torch.float32,
                     device="cuda")
    kw = dict(initial_state=d["initial_state"], output_final_state=True,
              cu_seqlens=d["cu_seqlens"], use_qk_l2norm_in_kernel=True,
              checkpoint_every_n_tokens=64, state_checkpoints=ck,
              checkpoint_cu_starts=d["checkpoint_cu_starts"])
    p, _, _ = api.make_params(d["q"], d["k"], d["v"], d["g"], d["beta"],
                              output=out, output_state=fin, **kw)
    ws = torch.empty(api.workspace_size(p), dtype=torch.uint8, device="cuda")

    def call():
        chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], output=out,
                               output_state=fin, status=st, workspace=ws, **kw)

    call()                                  # first call: per-device set-up
    torch.cuda.synchronize()
    ref_out, ref_fin, ref_ck = out.clone(), fin.clone(), ck.clone()
    out.zero_()
    fin.zero_()
    ck.zero_()
    busy, dt = _returns_while_busy(call)
    print("lengths", len(lengths), "call returned after %.1f us, stream busy: %s"
          % (dt * 1e6, busy), flush=True)
    assert busy
    assert int(st.item()) == 0
    assert torch.equal(out, ref_out)
    assert torch.equal(fin, ref_fin)
    assert torch.equal(ck, ref_ck)


def test_decode_returns_before_the_device_finishes():
    N, H, D = 64, 4, 128
    wl = W.make(71, [1] * N, H, H, H, D, "bf16", l2norm_in_kernel=True,
                init="pool", pool_size=80, init_std=0.3)
    d = tl.to_device(wl)
    pool0 = d["initial_state"].clone()
    pool = d["initial_state"].clone()
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        gated_delta_rule_decode(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                initial_state=pool, output_state=pool,
                                state_indices=d["state_indices"],
                                use_qk_l2norm_in_kernel=True, output=out)

    call()
    torch.cuda.synchronize()
    ref_out, ref_pool = out.clone(), pool.clone()
    pool.copy_(pool0)
    out.zero_()
    busy, dt = _returns_while_busy(call)
    print("decode call returned after %.1f us, stream busy: %s" % (dt * 1e6, busy), flush=True)
    assert busy
    assert torch.equal(out, ref_out)
    assert torch.equal(pool, ref_pool)
