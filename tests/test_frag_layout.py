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


# ---------------------------------------------------------------- K/Q chunk tiles in LDS
# The fused state pass keeps a chunk's K (and Q) tile in LDS row-major, 64 rows
# of dk values, with the 16-byte units of each row permuted by a row-dependent
# XOR so that both the MFMA operand reads and the transposing K^T reads hit
# distinct banks. These checks model the copy, both reads and the bank mapping
# on the CPU, mirroring the index arithmetic of k_state_output.

def _swz(row, upr):
    return ((((row & 3) << 1) | ((row >> 2) & 1) | (row & 8))) & (upr - 1)


def _copy_tile(K, dk):
    """LDS image (elements) of the tile after the 16-byte buffer-to-LDS copies:
    copy u, lane l lands at element 512 u + 8 l and fetches row 512/dk * u + l // upr,
    unit (l % upr) ^ swz(row)."""
    upr = dk // 8
    rpi = 512 // dk
    lds = np.full(64 * dk, -1.0)
    for u in range(dk // 8):
        for l in range(64):
            row = rpi * u + l // upr
            src_unit = (l % upr) ^ _swz(row, upr)
            lds[512 * u + 8 * l: 512 * u + 8 * l + 8] = K[row, 8 * src_unit: 8 * src_unit + 8]
    return lds


def _tr16_b64(lds, addrs):
    """ds_read_b64_tr_b16 over 16-lane groups: lane (qd, r') element e is element
    (r' & 3) of the 4-element row read by lane (qd, 4 e + (r' >> 2))."""
    src = np.stack([lds[a: a + 4] for a in addrs])
    out = np.zeros((64, 4))
    for l in range(64):
        qd, rp = l // 16, l % 16
        for e in range(4):
            out[l, e] = src[16 * qd + 4 * e + (rp >> 2), rp & 3]
    return out


def _max_bank_conflict(byte_addrs, nbytes, group):
    """Largest number of distinct addresses that share a 4-byte bank (32 banks)
    within each group of `group` consecutive lanes."""
    worst = 1
    for g0 in range(0, 64, group):
        banks = {}
        for a in byte_addrs[g0: g0 + group]:
            for b in range(a, a + nbytes, 4):
                banks.setdefault((b // 4) % 32, set()).add(b // 128)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def test_kq_tile_reads_fetch_the_right_elements():
    rng = np.random.default_rng(1)
    for dk in (32, 64, 128):
        upr = dk // 8
        K = rng.standard_normal((64, dk))
        lds = _copy_tile(K, dk)
        assert (lds >= -1e9).all()
        # A operand of K S / Q S: lane (qd, r) holds row 16 tb + r, dk 32 kp + 8 qd + e
        for tb in range(4):
            for kp in range(dk // 32):
                for l in range(64):
                    qd, r = l // 16, l % 16
                    row = 16 * tb + r
                    a = row * dk + 8 * ((4 * kp + qd) ^ _swz(row, upr))
                    assert np.array_equal(lds[a: a + 8], K[row, 32 * kp + 8 * qd: 32 * kp + 8 * qd + 8])
        # K^T operand: lane (qd, r') element e = K[16 tb + 4 qd + e][16 db + r']
        for db in range(dk // 16):
            for tb in range(4):
                addrs = []
                for l in range(64):
                    qd, j = l // 16, l % 16
                    row = 16 * tb + 4 * qd + (j >> 2)
                    unit = 2 * db + ((j & 3) >> 1)
                    addrs.append(row * dk + 8 * (unit ^ _swz(row, upr)) + 4 * (j & 1))
                got = _tr16_b64(lds, addrs)
                for l in range(64):
                    qd, rp = l // 16, l % 16
                    assert np.array_equal(got[l], K[16 * tb + 4 * qd: 16 * tb + 4 * qd + 4, 16 * db + rp])


def test_kq_tile_reads_are_bank_conflict_free_at_dk_64_and_128():
    for dk in (64, 128):
        upr = dk // 8
        frag = [(16 * 0 + l % 16) * dk * 2 + 16 * ((4 * 0 + l // 16) ^ _swz(l % 16, upr)) for l in range(64)]
        assert _max_bank_conflict(frag, 16, 8) == 1
        for db in range(dk // 16):
            tr = []
            for l in range(64):
                qd, j = l // 16, l % 16
                row = 4 * qd + (j >> 2)
                unit = 2 * db + ((j & 3) >> 1)
                tr.append(row * dk * 2 + 16 * (unit ^ _swz(row, upr)) + 8 * (j & 1))
            assert _max_bank_conflict(tr, 8, 16) == 1
