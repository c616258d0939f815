"""CPU checks of the fragment-layout unpacking used by the GPU parity tests."""
import numpy as np

from frag_layout import M_OF, unpack_pair, unpack_tile


def test_pair_order_is_a_permutation_per_lane_group():
    for qd in range(4):
        ms = sorted(M_OF[16 * qd].tolist())
        assert ms == sorted([4 * qd + e for e in range(4)] + [16 + 4 * qd + e for e in range(4)])
    assert sorted(set(M_OF.ravel().tolist())) == list(range(32))


def test_two_accumulator_tiles_are_a_pair_fragment_of_the_transpose():
    """Stacking tiles Y0 (rows 0..15) and Y1 (rows 16..31) of a 32 x 16 block B,
    lane-wise, gives the pair fragment of B^T: the identity the kernels use to
    feed an MFMA result into the next MFMA without moving data."""
    rng = np.random.default_rng(0)
    B = rng.standard_normal((32, 16))
    lane = np.arange(64)
    t0 = np.zeros((64, 4)); t1 = np.zeros((64, 4))
    for l in lane:
        qd, r = l // 16, l % 16
        for j in range(4):
            t0[l, j] = B[4 * qd + j, r]
            t1[l, j] = B[16 + 4 * qd + j, r]
    assert np.allclose(unpack_tile(t0), B[:16]) and np.allclose(unpack_tile(t1), B[16:])
    frag = np.concatenate([t0, t1], axis=1)
    assert np.allclose(unpack_pair(frag), B.T)
