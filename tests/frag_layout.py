"""Unpack the kernels' fragment-major intermediates into natural layouts.

Follows the layout contract stated in include/gdr.h (gdr_intermediates_t):
lane l = 16*qd + r; a pair fragment holds X[r][m(qd, e)] with
m(qd, e) = 4*qd + e (e < 4) or 16 + 4*qd + e - 4 (e >= 4); an accumulator tile
holds Y[4*qd + j][r].
"""
import numpy as np

_QD = np.arange(64) // 16
_R = np.arange(64) % 16
_E = np.arange(8)
M_OF = np.where(_E[None, :] < 4, 4 * _QD[:, None] + _E[None, :], 16 + 4 * _QD[:, None] + _E[None, :] - 4)  # [64, 8]


def unpack_pair(frag):
    """[..., 64, 8] -> X [..., 16, 32]."""
    frag = np.asarray(frag)
    X = np.zeros(frag.shape[:-2] + (16, 32), dtype=np.float64)
    X[..., _R[:, None], M_OF] = frag
    return X


def unpack_tile(tile):
    """[..., 64, 4] -> Y [..., 16, 16]."""
    tile = np.asarray(tile)
    Y = np.zeros(tile.shape[:-2] + (16, 16), dtype=np.float64)
    rows = 4 * _QD[:, None] + np.arange(4)[None, :]
    Y[..., rows, _R[:, None]] = tile
    return Y


def W_natural(W):
    """[NT, Nv, C/16, dk/32, 64, 8] -> [NT, Nv, C, dk] (rows = chunk position)."""
    X = unpack_pair(W)                                    # [NT, Nv, ntb, nkp, 16, 32]
    NT, Nv, ntb, nkp = X.shape[:4]
    return X.transpose(0, 1, 2, 4, 3, 5).reshape(NT, Nv, ntb * 16, nkp * 32)


def U_natural(U):
    """[NT, Nv, C/16, dv/16, 64, 4] -> [NT, Nv, C, dv]."""
    Y = unpack_tile(U)                                    # [NT, Nv, ntb, nnb, 16, 16]
    NT, Nv, ntb, nnb = Y.shape[:4]
    return Y.transpose(0, 1, 2, 4, 3, 5).reshape(NT, Nv, ntb * 16, nnb * 16)


def KT_natural(KT):
    """[NT, Nk, dk/16, ntp, 64, 8] -> K [NT, Nk, 32 ntp, dk] (ntp = max(1, C/32);
    with C = 16, positions 16..31 are the zero padding)."""
    X = unpack_pair(KT)                                   # [NT, Nk, ndb, ntp, 16(dk), 32(pos)]
    NT, Nk, ndb, ntp = X.shape[:4]
    KTn = X.transpose(0, 1, 2, 4, 3, 5).reshape(NT, Nk, ndb * 16, ntp * 32)
    return KTn.transpose(0, 1, 3, 2)


def H_natural(H):
    """[NT, Nv, dv/16, dk/32, 64, 8] -> S [NT, Nv, dk, dv]."""
    X = unpack_pair(H)                                    # [NT, Nv, nnb, nkp, 16(dv), 32(dk)]
    NT, Nv, nnb, nkp = X.shape[:4]
    ST = X.transpose(0, 1, 2, 4, 3, 5).reshape(NT, Nv, nnb * 16, nkp * 32)
    return ST.transpose(0, 1, 3, 2)


def VN_natural(VN):
    """[NT, Nv, dv/16, ntp, 64, 8] -> V_new [NT, Nv, 32 ntp, dv]."""
    X = unpack_pair(VN)                                   # [NT, Nv, nnb, ntp, 16(dv), 32(pos)]
    NT, Nv, nnb, ntp = X.shape[:4]
    VT = X.transpose(0, 1, 2, 4, 3, 5).reshape(NT, Nv, nnb * 16, ntp * 32)
    return VT.transpose(0, 1, 3, 2)


def chunk_rows_to_tokens(X, chunks, Ttot):
    """[NT, H, C, D] chunk-position rows -> [Ttot, H, D] token rows (valid rows only)."""
    NT, H, _, D = X.shape
    out = np.zeros((Ttot, H, D))
    for c, (_, s, L) in enumerate(chunks):
        out[s:s + L] = X[c, :, :L].transpose(1, 0, 2)
    return out


def pad_rows_are_zero(X, chunks):
    """True if every chunk position past a chunk's end holds zeros."""
    for c, (_, s, L) in enumerate(chunks):
        if np.any(X[c, :, L:] != 0):
            return False
    return True


T_PAIRS = ((0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1))


def T_natural(Tf):
    """[NT, Nv, 6, 64, 8] fp16 pair fragments -> [NT, Nv, 64, 64] (rows and
    columns = chunk positions; blocks not stored are zero). Used for T = A
    diag(beta) and for the score block P, which share the layout."""
    X = unpack_pair(np.asarray(Tf, dtype=np.float64))                # [NT, Nv, 6, 16, 32]
    NT, Nv = X.shape[:2]
    out = np.zeros((NT, Nv, 64, 64))
    for p, (tb, tp) in enumerate(T_PAIRS):
        out[:, :, tb * 16:(tb + 1) * 16, tp * 32:(tp + 1) * 32] = X[:, :, p]
    return out
