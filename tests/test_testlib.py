"""CPU checks of the parity helpers themselves: the block maxima catch a
localized error that the whole-tensor relative L2 lets through."""
import numpy as np

from tests import gdn_testlib as tl


def test_one_missing_chunk_hides_in_the_whole_tensor_but_not_in_the_blocks():
    # one 262144-token sequence (4096 chunks), one head: an output whose
    # every element is off by a relative 3e-3, except one 64-token chunk that
    # was never written (zeros).  The whole-tensor error stays under the
    # bf16 bar of 2e-2 (the chunk is 1/4096 of the tensor), the chunk's own
    # error is 1.
    rng = np.random.default_rng(0)
    T, H, D = 262144, 1, 16
    ref = rng.standard_normal((T, H, D))
    got = ref * (1.0 + 3e-3 * rng.standard_normal((T, H, D)))
    got[64 * 1234:64 * 1235] = 0.0
    assert tl.rel_l2(got, ref) < 2e-2
    cu = np.array([0, T])
    worst, where = tl.block_max_rel_l2(got, ref, tl.chunk_blocks(cu, H))
    assert worst > 0.99
    assert where == (slice(64 * 1234, 64 * 1235), 0)


def test_chunk_blocks_follow_sequence_starts():
    cu = np.array([0, 130, 150, 450, 450, 515])
    b = tl.chunk_blocks(cu, 2)
    starts = sorted({s.start for s, _ in b})
    assert starts == [0, 64, 128, 130, 150, 214, 278, 342, 406, 450, 514]
    assert all(s.stop - s.start <= 64 for s, _ in b)
    assert len(b) == 2 * len(starts)
    assert tl.sequence_blocks(cu) == [slice(0, 130), slice(130, 150), slice(150, 450),
                                      slice(450, 515)]


def test_block_error_floor_holds_small_blocks_to_the_tensor_scale():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((8, 4, 32))
    ref[5, 2] *= 1e-3                      # a block whose values nearly cancel
    x = ref + 1e-4 * rng.standard_normal(ref.shape)
    blocks = [(t, h) for t in range(8) for h in range(4)]
    e, _ = tl.block_max_rel_l2(x, ref, blocks)
    assert e < 1e-3                        # absolute 1e-4 error at scale 1
    x[3, 1] = 0.0                          # a zeroed block of typical scale
    e, where = tl.block_max_rel_l2(x, ref, blocks)
    assert where == (3, 1) and e > 0.8     # ||ref_b|| over the floor
