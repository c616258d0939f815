"""CPU pins for the fp64 oracle (both forms), independent of any GPU code.

Each test checks the oracle against something the pages or plain algebra fix,
not against a retyped copy of its own formula:

* WY identity of P (FLA DeltaNet article, section 2.1, Eq. 2) and of H
  (section 2.2, Eq. 3) against explicit Householder-type products;
* the solve (I + L) A = I against SciPy's triangular solver (section 2.3);
* token recurrence == chunked form for several chunk sizes (section 2.4);
* closed forms: beta = 0 gives pure decayed reads of S0; beta = 1 with unit
  keys stores v exactly (ChunkGatedDeltaRule page, section 1: the delta
  rule's write corrects the read); one token; null inputs;
* structure: linearity in (v, S0), continuation through the state,
  varlen packing == separate runs, GQA == repeated heads;
* a hand-worked two-token example (tests/golden/two_token_hand.json).
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import chunked_forward, recurrence
from oracle import chunked as ch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    r = np.sqrt(np.mean(b ** 2))
    return float(np.max(np.abs(a - b)) / (r if r > 0 else 1.0))


def rand_inputs(rng, T, Nk=1, Nv=1, dk=8, dv=4, gated=True, s0=True, unit_k=True, g_mean=2.0, N=1):
    q = rng.standard_normal((T, Nk, dk))
    k = rng.standard_normal((T, Nk, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Nv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Nv))))
    g = -np.log1p(np.exp(-(g_mean + rng.standard_normal((T, Nv))))) if gated else None
    S0 = 0.1 * rng.standard_normal((N, Nv, dk, dv)) if s0 else None
    return q, k, v, beta, g, S0


def explicit_P_H(Kc, Vc, beta, g):
    """Brute-force transition of one chunk: S_out = P S_in + H with
    P = prod_r exp(g_r)(I - beta_r k_r k_r^T) (newest factor on the left) and
    H = sum_i [prod_{j>i} exp(g_j)(I - beta_j k_j k_j^T)] beta_i k_i v_i^T."""
    n, dk = Kc.shape
    I = np.eye(dk)
    fac = [np.exp(g[r]) * (I - beta[r] * np.outer(Kc[r], Kc[r])) for r in range(n)]
    P = I.copy()
    for r in range(n):
        P = fac[r] @ P
    H = np.zeros((dk, Vc.shape[1]))
    for i in range(n):
        Pi = I.copy()
        for j in range(i + 1, n):
            Pi = fac[j] @ Pi
        H += Pi @ (beta[i] * np.outer(Kc[i], Vc[i]))
    return P, H


# --------------------------------------------------------------------- P1, P2
@pytest.mark.parametrize("dk,r", [(3, 2), (5, 4), (8, 8), (6, 8)])
def test_wy_identity_of_P(dk, r):
    """P^r = I - sum_{i<=r} k^i w^{i T} (Eq. 2), with w taken from the oracle's
    W = A diag(beta) K, against the explicit product of (I - beta k k^T)."""
    rng = np.random.default_rng(10 + dk + r)
    K = rng.standard_normal((r, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    beta = rng.uniform(0.05, 0.95, r)
    G = np.zeros(r)
    A = ch.unit_lower_inverse(ch.strict_lower_attn(K, beta, ch.decay_matrix(G)))
    W, _ = ch.wy_products(A, K, np.zeros((r, 1)), beta, G)
    for rr in range(1, r + 1):
        P_explicit, _ = explicit_P_H(K[:rr], np.zeros((rr, 1)), beta[:rr], np.zeros(rr))
        P_wy = np.eye(dk) - K[:rr].T @ W[:rr]
        assert rel(P_wy, P_explicit) < 1e-12


@pytest.mark.parametrize("dk,dv,r", [(4, 3, 3), (8, 5, 8), (6, 2, 7)])
def test_wy_identity_of_H(dk, dv, r):
    """H^r = sum_{i<=r} k^i u^{i T} (Eq. 3) with u from U = A diag(beta) V."""
    rng = np.random.default_rng(20 + dk + r)
    K = rng.standard_normal((r, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((r, dv))
    beta = rng.uniform(0.05, 0.95, r)
    G = np.zeros(r)
    A = ch.unit_lower_inverse(ch.strict_lower_attn(K, beta, ch.decay_matrix(G)))
    _, U = ch.wy_products(A, K, V, beta, G)
    for rr in range(1, r + 1):
        _, H_explicit = explicit_P_H(K[:rr], V[:rr], beta[:rr], np.zeros(rr))
        assert rel(K[:rr].T @ U[:rr], H_explicit) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 7, 16, 64])
def test_gated_chunk_transition_matches_explicit_product(n):
    """With gates, one chunk maps S_in to exp(G_last) S_in - Kt^T W S_in + Kt^T U
    with Kt = diag(exp(G_last - G)) K (formulas 3 and 6); compare the implied
    (P, H) with the explicit product of exp(g)(I - beta k k^T)."""
    rng = np.random.default_rng(30 + n)
    dk, dv = 6, 3
    K = rng.standard_normal((n, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((n, dv))
    beta = rng.uniform(0.05, 0.95, n)
    g = -rng.uniform(0.0, 0.5, n)
    G = ch.gate_cumsum(g)
    D = ch.decay_matrix(G)
    A = ch.unit_lower_inverse(ch.strict_lower_attn(K, beta, D))
    W, U = ch.wy_products(A, K, V, beta, G)
    P_explicit, H_explicit = explicit_P_H(K, V, beta, g)
    # Probe S_out as a function of S_in through the oracle's chunk step.
    Q = np.zeros((n, dk))
    S_zero = np.zeros((dk, dv))
    _, _, H_chunk = ch.chunk_state_and_output(S_zero, Q, K, W, U, G, D, 1.0)
    assert rel(H_chunk, H_explicit) < 1e-12
    for col in range(dk):
        E = np.zeros((dk, dv))
        E[col, 0] = 1.0
        _, _, S_out = ch.chunk_state_and_output(E, Q, K, W, U, G, D, 1.0)
        assert np.max(np.abs((S_out - H_chunk)[:, 0] - P_explicit[:, col])) < 1e-12


# ------------------------------------------------------------------------ P3
@pytest.mark.parametrize("n,seed", [(1, 0), (5, 1), (16, 2), (64, 3)])
def test_unit_lower_inverse_solves_system(n, seed):
    rng = np.random.default_rng(seed)
    L = np.tril(rng.uniform(-1, 1, (n, n)), -1)
    A = ch.unit_lower_inverse(L)
    I = np.eye(n)
    assert np.max(np.abs((I + L) @ A - I)) < 1e-10
    ref = scipy.linalg.solve_triangular(I + L, I, lower=True, unit_diagonal=True)
    assert np.max(np.abs(A - ref)) < 1e-10 * max(1.0, np.max(np.abs(ref)))
    assert np.allclose(np.triu(A, 1), 0) and np.allclose(np.diag(A), 1)


def test_gate_cumsum_and_decay_matrix():
    g = np.array([-0.5, -0.25, 0.0, -1.0])
    assert np.allclose(ch.gate_cumsum(g), np.cumsum(g))
    D = ch.decay_matrix(np.cumsum(g))
    assert np.allclose(np.triu(D, 1), 0)
    assert np.allclose(np.diag(D), 1)
    assert np.isclose(D[3, 0], np.exp(g[1] + g[2] + g[3]))   # decay over tokens 1..3
    assert np.isclose(D[2, 1], np.exp(0.0))


# ------------------------------------------------------------------------ P4
CASES = [
    # T, Nk, Nv, dk, dv, gated, s0
    (1, 1, 1, 8, 4, True, True),
    (63, 1, 2, 8, 4, True, True),
    (64, 2, 2, 16, 8, True, False),
    (65, 1, 1, 8, 8, False, True),
    (200, 2, 4, 16, 8, True, True),
    (1000, 1, 1, 16, 16, True, True),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("C", [1, 16, 32, 64])
def test_recurrence_equals_chunked(case, C):
    T, Nk, Nv, dk, dv, gated, s0 = case
    if T == 1000 and C < 16:
        pytest.skip("covered by the larger chunk sizes")
    rng = np.random.default_rng(T * 7 + C)
    q, k, v, beta, g, S0 = rand_inputs(rng, T, Nk, Nv, dk, dv, gated, s0)
    cu = np.array([0, T])
    o1, s1 = recurrence(q, k, v, beta, g, None, S0, cu)
    o2, s2 = chunked_forward(q, k, v, beta, g, None, S0, cu, chunk_size=C)
    assert rel(o2, o1) < 1e-10
    assert rel(s2, s1) < 1e-10


def test_recurrence_equals_chunked_varlen_gqa():
    rng = np.random.default_rng(5)
    lens = [0, 1, 64, 65, 130, 7]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, beta, g, S0 = rand_inputs(rng, T, 2, 4, 16, 8, True, True, N=len(lens))
    o1, s1 = recurrence(q, k, v, beta, g, 0.3, S0, cu)
    o2, s2 = chunked_forward(q, k, v, beta, g, 0.3, S0, cu, chunk_size=64)
    assert rel(o2, o1) < 1e-10 and rel(s2, s1) < 1e-10
    # zero-length sequence: no rows, S_T = S0
    assert np.allclose(s1[0], S0[0]) and np.allclose(s2[0], S0[0])


def test_literal_undecayed_read_is_not_the_chunk_form():
    """Reading of the decay placement: the literal printed recurrence (delta
    read from the undecayed state) disagrees with the chunk formulas once
    g != 0, and agrees with them when g == 0."""
    rng = np.random.default_rng(6)
    q, k, v, beta, g, S0 = rand_inputs(rng, 100, 1, 1, 8, 4, True, True)
    cu = np.array([0, 100])
    o_lit, _ = recurrence(q, k, v, beta, g, None, S0, cu, literal_undecayed_read=True)
    o_chk, _ = chunked_forward(q, k, v, beta, g, None, S0, cu)
    assert rel(o_lit, o_chk) > 1e-2
    o_lit0, s_lit0 = recurrence(q, k, v, beta, np.zeros_like(g), None, S0, cu, literal_undecayed_read=True)
    o_chk0, s_chk0 = chunked_forward(q, k, v, beta, np.zeros_like(g), None, S0, cu)
    assert rel(o_lit0, o_chk0) < 1e-10 and rel(s_lit0, s_chk0) < 1e-10


# ------------------------------------------------------------------------ P5
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_beta_zero_gives_decayed_reads_of_S0(form):
    rng = np.random.default_rng(7)
    T = 150
    q, k, v, beta, g, S0 = rand_inputs(rng, T, 1, 2, 8, 4, True, True)
    beta = np.zeros_like(beta)
    cu = np.array([0, T])
    scale = 0.7
    fn = recurrence if form == "recurrence" else chunked_forward
    o, ST = fn(q, k, v, beta, g, scale, S0, cu)
    for h in range(2):
        cg = np.cumsum(g[:, h])                   # cumulative across chunk boundaries
        expect = scale * np.exp(cg)[:, None] * (q[:, 0] @ S0[0, h])
        assert rel(o[:, h], expect) < 1e-12
        assert rel(ST[0, h], np.exp(cg[-1]) * S0[0, h]) < 1e-12


# ------------------------------------------------------------------------ P6
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_orthonormal_keys_store_v_exactly(form):
    rng = np.random.default_rng(8)
    dk, dv, T = 16, 5, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][:, None, :]                          # T orthonormal keys
    v = rng.standard_normal((T, 1, dv))
    beta = np.ones((T, 1))
    cu = np.array([0, T])
    fn = recurrence if form == "recurrence" else chunked_forward
    o, ST = fn(k, k, v, beta, np.zeros((T, 1)), 1.0, None, cu)
    assert np.max(np.abs(k[:, 0] @ ST[0, 0] - v[:, 0])) < 1e-12
    assert np.max(np.abs(o[:, 0] - v[:, 0])) < 1e-12


# ------------------------------------------------------------------------ P7
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_unit_key_beta_one_stores_v_under_any_gate(form):
    """beta = 1 and |k| = 1: after token t, k_t^T S_t = v_t for any g and S0.
    Holds only when the delta is read from the decayed state."""
    rng = np.random.default_rng(9)
    T = 140
    q, k, v, beta, g, S0 = rand_inputs(rng, T, 1, 1, 8, 4, True, True, g_mean=0.5)
    beta = np.ones_like(beta)
    cu = np.array([0, T])
    fn = recurrence if form == "recurrence" else chunked_forward
    o, _ = fn(k, k, v, beta, g, 1.0, S0, cu)         # q = k reads k_t^T S_t
    assert np.max(np.abs(o - v)) < 1e-11
    o_lit, _ = recurrence(k, k, v, beta, g, 1.0, S0, cu, literal_undecayed_read=True)
    assert np.max(np.abs(o_lit - v)) > 1e-3


# ------------------------------------------------------------------------ P8
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_single_token_closed_form(form):
    rng = np.random.default_rng(11)
    q, k, v, beta, g, S0 = rand_inputs(rng, 1, 1, 1, 8, 4, True, True)
    fn = recurrence if form == "recurrence" else chunked_forward
    scale = 0.9
    o, ST = fn(q, k, v, beta, g, scale, S0, np.array([0, 1]))
    a, b = np.exp(g[0, 0]), beta[0, 0]
    S, kk, qq, vv = S0[0, 0], k[0, 0], q[0, 0], v[0, 0]
    delta = b * (vv - a * (S.T @ kk))
    S_expect = a * S + np.outer(kk, delta)
    o_expect = scale * (a * (qq @ S) + (qq @ kk) * delta)
    assert rel(ST[0, 0], S_expect) < 1e-13
    assert rel(o[0, 0], o_expect) < 1e-13


# ------------------------------------------------------------------------ P9
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_linear_in_v_and_S0(form):
    rng = np.random.default_rng(12)
    T = 130
    q, k, v1, beta, g, S1 = rand_inputs(rng, T, 1, 2, 8, 4, True, True)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    cu = np.array([0, T])
    fn = recurrence if form == "recurrence" else chunked_forward
    a, b = 0.7, -1.3
    oa, sa = fn(q, k, v1, beta, g, None, S1, cu)
    ob, sb = fn(q, k, v2, beta, g, None, S2, cu)
    oc, sc = fn(q, k, a * v1 + b * v2, beta, g, None, a * S1 + b * S2, cu)
    assert rel(oc, a * oa + b * ob) < 1e-11
    assert rel(sc, a * sa + b * sb) < 1e-11


# ----------------------------------------------------------------------- P10
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
@pytest.mark.parametrize("T1", [64, 100])
def test_continuation_through_state(form, T1):
    rng = np.random.default_rng(13)
    T = 230
    q, k, v, beta, g, S0 = rand_inputs(rng, T, 1, 1, 8, 4, True, True)
    fn = recurrence if form == "recurrence" else chunked_forward
    o, ST = fn(q, k, v, beta, g, None, S0, np.array([0, T]))
    oa, Sa = fn(q[:T1], k[:T1], v[:T1], beta[:T1], g[:T1], None, S0, np.array([0, T1]))
    ob, Sb = fn(q[T1:], k[T1:], v[T1:], beta[T1:], g[T1:], None, Sa, np.array([0, T - T1]))
    assert rel(np.concatenate([oa, ob]), o) < 1e-11
    assert rel(Sb, ST) < 1e-11


# ----------------------------------------------------------------------- P11
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_varlen_equals_separate_runs(form):
    rng = np.random.default_rng(14)
    lens = [3, 70, 64, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, beta, g, S0 = rand_inputs(rng, cu[-1], 1, 2, 8, 4, True, True, N=len(lens))
    fn = recurrence if form == "recurrence" else chunked_forward
    o, ST = fn(q, k, v, beta, g, None, S0, cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, Sn = fn(q[s:e], k[s:e], v[s:e], beta[s:e], g[s:e], None, S0[n:n + 1], np.array([0, e - s]))
        assert rel(o[s:e], on) < 1e-12 and rel(ST[n], Sn[0]) < 1e-12


@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_gqa_equals_repeated_heads(form):
    rng = np.random.default_rng(15)
    T, Nk, Nv = 90, 2, 6
    q, k, v, beta, g, S0 = rand_inputs(rng, T, Nk, Nv, 8, 4, True, True)
    fn = recurrence if form == "recurrence" else chunked_forward
    cu = np.array([0, T])
    o, ST = fn(q, k, v, beta, g, None, S0, cu)
    rep = Nv // Nk
    qr, kr = np.repeat(q, rep, axis=1), np.repeat(k, rep, axis=1)   # consecutive V-heads share
    o2, ST2 = fn(qr, kr, v, beta, g, None, S0, cu)
    assert rel(o, o2) < 1e-12 and rel(ST, ST2) < 1e-12


# ----------------------------------------------------------------------- P12
@pytest.mark.parametrize("form", ["recurrence", "chunked"])
def test_null_inputs_give_zero(form):
    rng = np.random.default_rng(16)
    q, k, v, beta, g, _ = rand_inputs(rng, 80, 1, 1, 8, 4, True, False)
    fn = recurrence if form == "recurrence" else chunked_forward
    o, ST = fn(q, k, np.zeros_like(v), beta, g, None, None, np.array([0, 80]))
    assert np.all(o == 0) and np.all(ST == 0)


def test_ungated_equals_zero_gate():
    rng = np.random.default_rng(17)
    q, k, v, beta, g, S0 = rand_inputs(rng, 70, 1, 1, 8, 4, True, True)
    for fn in (recurrence, chunked_forward):
        oa, sa = fn(q, k, v, beta, None, None, S0, np.array([0, 70]))
        ob, sb = fn(q, k, v, beta, np.zeros_like(g), None, S0, np.array([0, 70]))
        assert np.array_equal(oa, ob) and np.array_equal(sa, sb)


# -------------------------------------------------------------- golden file
def test_hand_worked_two_token_example():
    with open(os.path.join(GOLDEN, "two_token_hand.json")) as f:
        gold = json.load(f)
    x = gold["inputs"]
    q = np.array(x["q"])[:, None, :]
    k = np.array(x["k"])[:, None, :]
    v = np.array(x["v"])[:, None, :]
    beta = np.array(x["beta"])[:, None]
    g = np.array(x["g"])[:, None]
    S0 = np.array(x["S0"])[None, None]
    cu = np.array([0, 2])
    exp_o = np.array(gold["expected"]["o"])
    exp_S = np.array(gold["expected"]["S_T"])
    for fn in (recurrence, chunked_forward):
        o, ST = fn(q, k, v, beta, g, x["scale"], S0, cu)
        assert np.max(np.abs(o[:, 0] - exp_o)) < 1e-12
        assert np.max(np.abs(ST[0, 0] - exp_S)) < 1e-12
    o_lit, _ = recurrence(q, k, v, beta, g, x["scale"], S0, cu, literal_undecayed_read=True)
    assert abs(o_lit[0, 0, 0] - gold["expected"]["o_literal_undecayed_token0"]) < 1e-12


def test_intermediates_layout_and_consistency():
    """The chunked oracle's intermediates obey the layout it documents."""
    rng = np.random.default_rng(18)
    lens = [100, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, beta, g, S0 = rand_inputs(rng, cu[-1], 1, 2, 8, 4, True, True, N=2)
    r = chunked_forward(q, k, v, beta, g, None, S0, cu, intermediates=True)
    assert r["chunks"].tolist() == [[0, 0, 64], [0, 64, 36], [1, 100, 64]]
    assert np.allclose(r["h"][0], S0[0]) and np.allclose(r["h"][2], S0[1])
    # G restarts at every chunk start
    assert np.allclose(r["G"][64], g[64]) and np.allclose(r["G"][100], g[100])
    # A rows of the tail chunk are zero past the chunk end and above the diagonal
    A_tail = r["A"][64:100]
    assert np.allclose(A_tail[:, :, 36:], 0)
    for i in range(36):
        assert np.allclose(A_tail[i, :, i + 1:], 0) and np.allclose(A_tail[i, :, i], 1)


# ---------------------------------------------------------------- L2 normalisation of q, k (token-by-token option)
def test_l2_normalize_pins():
    from oracle import l2_normalize
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 3, 64))
    # eps = 0: the textbook unit vector x / ||x|| (NumPy's norm as an independent routine)
    ref = x / np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.max(np.abs(l2_normalize(x, eps=0.0) - ref)) < 1e-15
    # unit length, and invariant to positive scaling
    assert np.allclose(np.linalg.norm(l2_normalize(x, eps=0.0), axis=-1), 1.0, atol=1e-15)
    assert np.max(np.abs(l2_normalize(7.5 * x, eps=0.0) - l2_normalize(x, eps=0.0))) < 1e-15
    # default eps: the norm falls short of one by eps / (2 ||x||^2) to first order
    n2 = np.sum(x * x, axis=-1)
    got = np.linalg.norm(l2_normalize(x), axis=-1)
    assert np.allclose(got, 1.0 - 1e-6 / (2 * n2), rtol=0, atol=1e-13)
    # a zero vector stays zero (no division by zero)
    z = l2_normalize(np.zeros((2, 8)))
    assert np.all(z == 0.0)
