"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of the oracle on the CPU (a textual
edit of the C recurrence, compiled into a temporary library, or a monkeypatched
step of the NumPy chunked form) and checks that at least one pin fails. The
pins used here are the same closed forms and cross-form checks as in
test_oracle_pins.py.
"""
import json
import os

import numpy as np
import pytest

import oracle.chunked as ch
from oracle import chunked_forward, recurrence
from oracle.recurrence import compile_source

HERE = os.path.dirname(__file__)
SRC = os.path.join(os.path.dirname(HERE), "oracle", "recurrence.c")


def rel(a, b):
    r = np.sqrt(np.mean(np.asarray(b) ** 2))
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / (r if r > 0 else 1.0))


def _inputs(seed, T, Nk=1, Nv=1, dk=8, dv=4, g_mean=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Nk, dk))
    k = rng.standard_normal((T, Nk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Nv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Nv))))
    g = -np.log1p(np.exp(-(g_mean + rng.standard_normal((T, Nv)))))
    S0 = 0.1 * rng.standard_normal((1, Nv, dk, dv))
    return q, k, v, beta, g, S0


def pin_failures(fn, other):
    """Run a battery of pins on form ``fn``; return the names of those that fail.
    ``other`` is the independent form used for the cross-form pin."""
    bad = []
    # golden hand-worked example
    with open(os.path.join(HERE, "golden", "two_token_hand.json")) as f:
        gold = json.load(f)
    x = gold["inputs"]
    o, ST = fn(np.array(x["q"])[:, None], np.array(x["k"])[:, None], np.array(x["v"])[:, None],
               np.array(x["beta"])[:, None], np.array(x["g"])[:, None], x["scale"],
               np.array(x["S0"])[None, None], np.array([0, 2]))
    if np.max(np.abs(o[:, 0] - np.array(gold["expected"]["o"]))) > 1e-9 or \
            np.max(np.abs(ST[0, 0] - np.array(gold["expected"]["S_T"]))) > 1e-9:
        bad.append("golden")
    # beta = 0: decayed reads of S0
    q, k, v, beta, g, S0 = _inputs(1, 150, Nv=2)
    o, ST = fn(q, k, v, np.zeros_like(beta), g, 0.7, S0, np.array([0, 150]))
    for h in range(2):
        cg = np.cumsum(g[:, h])
        if rel(o[:, h], 0.7 * np.exp(cg)[:, None] * (q[:, 0] @ S0[0, h])) > 1e-9:
            bad.append("beta0")
            break
    # beta = 1, unit keys: k_t^T S_t = v_t
    q, k, v, beta, g, S0 = _inputs(2, 140, g_mean=0.5)
    o, _ = fn(k, k, v, np.ones_like(beta), g, 1.0, S0, np.array([0, 140]))
    if np.max(np.abs(o - v)) > 1e-9:
        bad.append("store_exact")
    # single-token closed form
    q, k, v, beta, g, S0 = _inputs(3, 1)
    o, ST = fn(q, k, v, beta, g, 0.9, S0, np.array([0, 1]))
    a, b = np.exp(g[0, 0]), beta[0, 0]
    d = b * (v[0, 0] - a * (S0[0, 0].T @ k[0, 0]))
    if rel(ST[0, 0], a * S0[0, 0] + np.outer(k[0, 0], d)) > 1e-9 or \
            rel(o[0, 0], 0.9 * (a * (q[0, 0] @ S0[0, 0]) + (q[0, 0] @ k[0, 0]) * d)) > 1e-9:
        bad.append("one_token")
    # cross-form agreement, GQA + varlen + tail chunks
    q, k, v, beta, g, S0 = _inputs(4, 200, Nk=2, Nv=4)
    S0 = np.concatenate([S0, 0.5 * S0], axis=0)
    cu = np.array([0, 70, 200])
    o1, s1 = fn(q, k, v, beta, g, None, S0, cu)
    o2, s2 = other(q, k, v, beta, g, None, S0, cu)
    if rel(o1, o2) > 1e-9 or rel(s1, s2) > 1e-9:
        bad.append("cross_form")
    # GQA == repeated heads
    o3, _ = fn(np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1), v, beta, g, None, S0, cu)
    if rel(o1, o3) > 1e-9:
        bad.append("gqa")
    return bad


def test_unmutated_oracle_passes_battery():
    assert pin_failures(recurrence, chunked_forward) == []
    assert pin_failures(chunked_forward, recurrence) == []


C_MUTATIONS = {
    "dropped_beta": ("read[j] = bt * (vt[j] - read_factor * read[j]);",
                     "read[j] = (vt[j] - read_factor * read[j]);"),
    "gate_sign": ("exp(g[(size_t)t * Nv + h])", "exp(-g[(size_t)t * Nv + h])"),
    "undecayed_read": ("literal_undecayed_read ? 1.0 : at;", "1.0;"),
    "wrong_outer_operand": ("S[(size_t)i * dv + j] += kt[i] * read[j];",
                            "S[(size_t)i * dv + j] += qt[i] * read[j];"),
    "head_map_mod": ("const int32_t kh = h / group;", "const int32_t kh = h % Nk;"),
    "dropped_scale": ("ot[j] = scale * acc;", "ot[j] = acc;"),
    "transposed_read": ("read[j] += kt[i] * S[(size_t)i * dv + j];",
                        "read[j] += kt[i] * S[(size_t)j * dv + i];"),
}


@pytest.mark.parametrize("name", sorted(C_MUTATIONS))
def test_recurrence_mutation_is_caught(name, tmp_path):
    before, after = C_MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, name
    mutated = tmp_path / "rec_mut.c"
    mutated.write_text(src.replace(before, after))
    lib = compile_source(str(mutated), str(tmp_path / ("librec_%s.so" % name)))

    def fn(*a, **kw):
        return recurrence(*a, lib_path=lib, **kw)
    assert pin_failures(fn, chunked_forward), name


PY_MUTATIONS = {
    # the output's intra-chunk mask drops the diagonal
    "mask_without_diagonal": ("decay_matrix", lambda orig: (lambda G: np.tril(orig(G), -1))),
    # gamma in formula (1) read as "decayed to the chunk end"
    "w_decay_to_chunk_end": ("wy_products", lambda orig: (
        lambda A, K, V, b, G: (A @ ((b * np.exp(G[-1] - G))[:, None] * K), A @ (b[:, None] * V)))),
    # transposed inverse
    "transposed_inverse": ("unit_lower_inverse", lambda orig: (lambda L: orig(L).T)),
    # S_out forgets to decay S_in
    "state_not_decayed": ("chunk_state_and_output", lambda orig: (
        lambda S, Q, K, W, U, G, D, sc: (lambda r: (r[0], r[1], r[2] - (np.exp(G[-1]) - 1.0) * S))(
            orig(S, Q, K, W, U, G, D, sc)))),
    # beta dropped from the A build
    "attn_without_beta": ("strict_lower_attn", lambda orig: (lambda K, b, D: orig(K, np.ones_like(b), D))),
    # exclusive instead of inclusive prefix sum
    "exclusive_cumsum": ("gate_cumsum", lambda orig: (lambda g: orig(g) - g)),
    # the recursive correction of the A rows is skipped (first-order inverse I - L)
    "no_recursive_correction": ("unit_lower_inverse", lambda orig: (lambda L: np.eye(len(L)) - L)),
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_chunked_mutation_is_caught(name, monkeypatch):
    attr, make = PY_MUTATIONS[name]
    orig = getattr(ch, attr)
    monkeypatch.setattr(ch, attr, make(orig))
    assert pin_failures(chunked_forward, recurrence), name
