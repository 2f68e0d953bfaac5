"""GPU parity over seeded random configurations, through the C ABI.

Each case draws (from its own seed) a batch of 1-7 sequences with lengths in
[0, 300] (ragged tails and empty sequences included), a legal head sharing,
a head size, an input dtype, a state arrangement (none, one per sequence, or a
pool read and written in place), the state dtypes, gates or none, in-kernel
normalisation or not, and checkpoints or none; the HIP path must match the
oracle's token recurrence to the same bars as the named configurations.
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


HEADS = [(2, 2, 2), (4, 2, 2), (2, 2, 4), (3, 3, 3), (1, 1, 4), (4, 1, 1)]


def _case(seed, many=False):
    rng = np.random.default_rng(7000 + seed)
    # many: batches of 33-50 sequences, which with the larger head counts and
    # sizes take the state pass's two-tile workgroups and longest-first order
    n = int(rng.integers(33, 51)) if many else int(rng.integers(1, 8))
    lengths = [int(x) for x in rng.integers(0, 301, size=n)]
    if rng.random() < 0.3:
        lengths[int(rng.integers(0, n))] = 0
    hq, hk, hv = HEADS[int(rng.integers(0, len(HEADS)))]
    D = int(rng.choice([32, 64, 128]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    kind = str(rng.choice(["none", "seq", "pool"]))
    sdt = ["f32", "bf16", "f16", "e4m3", "e5m2"]
    kw = dict(l2norm_in_kernel=bool(rng.random() < 0.7), gates=bool(rng.random() < 0.85),
              init_std=0.1)
    if kind == "seq":
        kw.update(init="seq", init_dtype=str(rng.choice(sdt)))
    elif kind == "pool":
        # in place: one dtype for reading and writing the pool
        pdt = str(rng.choice(sdt))
        kw.update(init="pool", pool_size=n + int(rng.integers(0, 5)), in_place_pool=True,
                  init_dtype=pdt, final_state_dtype=pdt)
    if kind != "pool":
        kw.update(final_state_dtype=str(rng.choice(sdt)))
    if rng.random() < 0.4:
        kw.update(checkpoint_every=int(rng.choice([64, 128])),
                  checkpoint_dtype=str(rng.choice(["f32", "bf16", "e4m3"])))
    if not kw["l2norm_in_kernel"]:
        kw["normalise_in_generator"] = True
    wl = W.make(8000 + seed, lengths, hq, hk, hv, D, dtype,
                name=("random_many%d" if many else "random%d") % seed, **kw)
    return wl


@pytest.mark.parametrize("seed,many", [(s, False) for s in range(16)] +
                         [(s, True) for s in range(100, 108)])
def test_random_config(seed, many):
    wl = _case(seed, many)
    gpu = tl.run_gpu(wl, status=True)
    assert gpu["status"] == 0
    orc = tl.run_oracle(wl)
    errs, _ = tl.compare(wl, gpu, orc)
    bars = tl.bars(wl)
    print(wl.name, wl.dtype, wl.D, wl.lengths, {k: "%.3e" % v for k, v in errs.items()},
          "bars", bars, flush=True)
    for k, e in errs.items():
        assert e <= bars[k], (k, e, bars[k])
    if wl.state_indices is not None:
        idx = set(int(r) for r in wl.state_indices)
        rows = gpu["pool_before"].shape[0]
        others = [r for r in range(rows) if r not in idx]
        np.testing.assert_array_equal(gpu["final"][others], gpu["pool_before"][others])
