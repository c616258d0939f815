"""Oracle: chunked (WY / UT form) gated delta-rule forward in fp64, NumPy.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the bench's
CPU-baseline leg; never by the product path, with which it shares no code.

This is the second, independent CPU form of the method. It does not call the
token recurrence; it follows the chunk algorithm step by step, in the order
and notation of the pages, one (sequence, V-head, chunk) at a time:

  G      chunk-local inclusive prefix sum of the log gates g
         (ChunkGatedDeltaRule page, section 3; GLA notes, forward step 1)
  D      D_ij = exp(G_i - G_j) for i >= j, else 0   (same page, section 3)
  L      strictly lower part of beta_i (k_i . k_j) D_ij
         (FLA DeltaNet article, section 2.3 and 3.1; ChunkGatedDeltaRule
         page, section 3.1 "direct term")
  A      (I + L)^-1, the inverse of the unit lower-triangular matrix the
         pages define (FLA DeltaNet article, section 2.3, the matrix T =
         (I + tril(diag(beta) K K^T, -1))^-1 diag(beta) with the decay of the
         gated form; ChunkGatedDeltaRule page, section 3.1 and formulas (1)-(2),
         where A multiplies the beta-scaled rows). Solved here from its
         definition (I + L) A = I, one column at a time by forward substitution
  W      A diag(beta * exp(G)) K        formula (1), "k_cumdecay"
  U      A diag(beta) V                 formula (2), "value_new"
  h      S_in, the state entering the chunk
  V_new  U - W S_in                     formula (3)
  O      scale [diag(exp(G)) Q S_in + (Q K^T (.) D) V_new]   formulas (4), (5)
         (the diagonal is kept: the output reads the state after its own write)
  S_out  exp(G_last) S_in + (diag(exp(G_last - G)) K)^T V_new   formula (6)

For the ungated rule (g absent) G is 0 and every exponential factor is 1; the
formulas then reduce to the FLA DeltaNet article's section 2.4.

Readings where the pages are silent or garbled (all consistent with the token
recurrence under the "forget first" reading):
  * the gamma in formula (1) is exp(G_i), cumulative from the chunk start;
  * chunks restart at every sequence start; the last chunk of a sequence may be
    shorter than C, and G_last is then the last valid token's prefix sum;
  * GQA: V-head h uses q/k head h // (Nv / Nk).

Layouts of the returned intermediates (natural, row-major):
  G [Ttot, Nv]; A [Ttot, Nv, C] (row of the token's position in its chunk,
  columns = positions in the chunk, zero above the diagonal and past the chunk
  end); W [Ttot, Nv, dk]; U, V_new [Ttot, Nv, dv]; h [NT, Nv, dk, dv] with
  chunks numbered sequence by sequence in token order; o [Ttot, Nv, dv];
  S_T [N, Nv, dk, dv].
"""
from __future__ import annotations

import numpy as np


def gate_cumsum(g_chunk: np.ndarray) -> np.ndarray:
    """G_i = sum_{j <= i} g_j inside one chunk (inclusive, chunk-local)."""
    G = np.zeros_like(g_chunk)
    acc = 0.0
    for i in range(len(g_chunk)):
        acc = acc + g_chunk[i]
        G[i] = acc
    return G


def decay_matrix(G: np.ndarray) -> np.ndarray:
    """D_ij = exp(G_i - G_j) for i >= j, 0 above the diagonal.

    Only non-positive exponents are formed (G is non-increasing when g <= 0).
    """
    L = len(G)
    D = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            D[i, j] = np.exp(G[i] - G[j])
    return D


def strict_lower_attn(Kc: np.ndarray, beta: np.ndarray, D: np.ndarray) -> np.ndarray:
    """L_ij = beta_i (k_i . k_j) D_ij for i > j, else 0."""
    KK = Kc @ Kc.T
    L = beta[:, None] * KK * D
    return np.tril(L, -1)


def unit_lower_inverse(Lmat: np.ndarray) -> np.ndarray:
    """A = (I + L)^-1 for strictly lower-triangular L.

    A is defined by (I + L) A = I. Column j of A solves (I + L) x = e_j; since
    I + L is unit lower-triangular, row i of that system reads
    x_i + sum_{m < i} L_im x_m = [i == j], so the entries follow in increasing
    i by forward substitution (entries above the diagonal come out zero).
    """
    n = Lmat.shape[0]
    A = np.zeros((n, n))
    for j in range(n):
        x = np.zeros(n)
        for i in range(n):
            rhs = 1.0 if i == j else 0.0
            x[i] = rhs - float(np.dot(Lmat[i, :i], x[:i]))
        A[:, j] = x
    return A


def wy_products(A, Kc, Vc, beta, G):
    """W = A diag(beta exp(G)) K (formula 1), U = A diag(beta) V (formula 2)."""
    W = A @ ((beta * np.exp(G))[:, None] * Kc)
    U = A @ (beta[:, None] * Vc)
    return W, U


def chunk_state_and_output(S_in, Qc, Kc, W, U, G, D, scale):
    """Formulas (3)-(6): V_new, O and S_out for one chunk."""
    V_new = U - W @ S_in
    O_inter = np.exp(G)[:, None] * (Qc @ S_in)
    O_intra = ((Qc @ Kc.T) * D) @ V_new
    O = scale * (O_inter + O_intra)
    G_last = G[-1]
    S_out = np.exp(G_last) * S_in + (np.exp(G_last - G)[:, None] * Kc).T @ V_new
    return V_new, O, S_out


def chunked_forward(q, k, v, beta, g=None, scale=None, S0=None, cu_seqlens=None,
                    chunk_size: int = 64, intermediates: bool = False):
    """Chunked forward in fp64.

    q, k: [Ttot, Nk, dk] (or [B, T, Nk, dk] without cu_seqlens); v: [.., Nv, dv];
    beta, g: [.., Nv]; S0: [N, Nv, dk, dv] or None; cu_seqlens: [N+1] or None.
    Returns (o, S_T) or, with intermediates=True, a dict that also holds
    G, A, W, U, h, V_new and the chunk table (seq, start, length).
    """
    f = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, beta, g, S0 = map(f, (q, k, v, beta, g, S0))
    lead = q.shape[:-2]
    if cu_seqlens is None:
        B, T = (q.shape[0], q.shape[1]) if q.ndim == 4 else (1, q.shape[0])
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    Nk, dk = q.shape[-2:]
    Nv, dv = v.shape[-2:]
    Ttot = int(np.prod(lead))
    N = len(cu) - 1
    group = Nv // Nk
    C = int(chunk_size)
    q, k = q.reshape(Ttot, Nk, dk), k.reshape(Ttot, Nk, dk)
    v, beta = v.reshape(Ttot, Nv, dv), beta.reshape(Ttot, Nv)
    g = np.zeros((Ttot, Nv)) if g is None else g.reshape(Ttot, Nv)
    if scale is None:
        scale = dk ** -0.5

    chunks = []                                   # (seq, start, length), sequence-major
    for n in range(N):
        for s in range(int(cu[n]), int(cu[n + 1]), C):
            chunks.append((n, s, min(C, int(cu[n + 1]) - s)))
    NT = len(chunks)

    o = np.zeros((Ttot, Nv, dv))
    S_T = np.zeros((N, Nv, dk, dv))
    if intermediates:
        G_all = np.zeros((Ttot, Nv))
        A_all = np.zeros((Ttot, Nv, C))
        W_all = np.zeros((Ttot, Nv, dk))
        U_all = np.zeros((Ttot, Nv, dv))
        Vn_all = np.zeros((Ttot, Nv, dv))
        h_all = np.zeros((NT, Nv, dk, dv))

    for h in range(Nv):
        kh = h // group
        state = {n: (S0[n, h].copy() if S0 is not None else np.zeros((dk, dv))) for n in range(N)}
        for c, (n, s, Lc) in enumerate(chunks):
            e = s + Lc
            Qc, Kc, Vc = q[s:e, kh], k[s:e, kh], v[s:e, h]
            bc = beta[s:e, h]
            G = gate_cumsum(g[s:e, h])
            D = decay_matrix(G)
            Lm = strict_lower_attn(Kc, bc, D)
            A = unit_lower_inverse(Lm)
            W, U = wy_products(A, Kc, Vc, bc, G)
            S_in = state[n]
            V_new, O, S_out = chunk_state_and_output(S_in, Qc, Kc, W, U, G, D, scale)
            o[s:e, h] = O
            if intermediates:
                G_all[s:e, h] = G
                A_all[s:e, h, :Lc] = A
                W_all[s:e, h] = W
                U_all[s:e, h] = U
                Vn_all[s:e, h] = V_new
                h_all[c, h] = S_in
            state[n] = S_out
        for n in range(N):
            S_T[n, h] = state[n]

    o = o.reshape(*lead, Nv, dv)
    if not intermediates:
        return o, S_T
    return dict(o=o, S_T=S_T, G=G_all, A=A_all, W=W_all, U=U_all, V_new=Vn_all, h=h_all,
                chunks=np.asarray(chunks, dtype=np.int64).reshape(-1, 3))
