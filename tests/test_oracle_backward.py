"""CPU pins for the backward oracle (``oracle.recurrence_backward``).

The analytic gradients are checked against central finite differences of the
fp64 forward (``oracle.recurrence``, itself pinned in test_oracle_pins.py) for
every input element, with L = sum(do * o) + sum(dS_T * S_T) for random do and
dS_T. A dropped term, a wrong sign or a transposed operand in any gradient
moves that gradient by far more than the difference quotient's error (about
1e-9 here). Cases: GQA with variable lengths and an empty sequence, an
initial state and a final-state gradient; the ungated rule; a strongly
decaying gate. Plus closed forms: beta = 0 gives dv = 0; one token from a zero
state has closed-form dv, dq and initial-state gradient. Planted mistakes in a
copy of the oracle (dropped term, wrong sign, wrong state, transposed operand,
missing decay) each fail the finite-difference pin.
"""
import numpy as np
import pytest

from oracle import recurrence, recurrence_backward


def problem(seed, lengths=(3, 0, 5), Nk=1, Nv=2, dk=3, dv=4, gated=True, g_mean=0.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    x = dict(
        q=rng.standard_normal((T, Nk, dk)),
        k=rng.standard_normal((T, Nk, dk)) * 0.5,
        v=rng.standard_normal((T, Nv, dv)),
        beta=rng.uniform(0.1, 0.9, (T, Nv)),
        g=(g_mean + 0.3 * rng.standard_normal((T, Nv))) if gated else None,
        S0=rng.standard_normal((N, Nv, dk, dv)) * 0.3,
    )
    w = dict(do=rng.standard_normal((T, Nv, dv)), dS_T=rng.standard_normal((N, Nv, dk, dv)))
    return x, cu, w


def loss(x, cu, w, scale):
    o, ST = recurrence(x["q"], x["k"], x["v"], x["beta"], x["g"], scale, x["S0"], cu)
    return float(np.sum(w["do"] * o) + np.sum(w["dS_T"] * ST))


def finite_difference(x, cu, w, scale, name, h=1e-6):
    base = x[name]
    grad = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        xp = dict(x)
        xp[name] = base.copy()
        xp[name][idx] += h
        lp = loss(xp, cu, w, scale)
        xp[name][idx] -= 2 * h
        lm = loss(xp, cu, w, scale)
        grad[idx] = (lp - lm) / (2 * h)
    return grad


NAMES = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "g": "dg", "S0": "dS0"}


@pytest.mark.parametrize("case", ["gqa_varlen", "ungated", "strong_decay", "mha_d5"])
def test_backward_matches_finite_differences(case):
    kw = dict(gqa_varlen={}, ungated=dict(gated=False), strong_decay=dict(g_mean=-2.0),
              mha_d5=dict(lengths=(4, 2), Nk=2, Nv=2, dk=5, dv=2))[case]
    x, cu, w = problem(1 + len(case), **kw)
    scale = 0.7
    grads = recurrence_backward(x["q"], x["k"], x["v"], x["beta"], x["g"], scale, x["S0"], cu, w["do"], w["dS_T"])
    for name, key in NAMES.items():
        if x[name] is None:
            assert grads[key] is None
            continue
        fd = finite_difference(x, cu, w, scale, name)
        err = np.max(np.abs(grads[key] - fd))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), (case, name, err)


def test_zero_beta_has_no_value_gradient():
    """beta = 0: v never enters the state, so dv = 0; the state only decays, and
    dbeta_t = du . (v_t - p_t) is still defined."""
    x, cu, w = problem(11)
    x["beta"] = np.zeros_like(x["beta"])
    grads = recurrence_backward(x["q"], x["k"], x["v"], x["beta"], x["g"], 1.0, x["S0"], cu, w["do"], w["dS_T"])
    assert np.all(grads["dv"] == 0)
    assert np.max(np.abs(grads["dbeta"])) > 0
    fd = finite_difference(x, cu, w, 1.0, "beta")
    assert np.max(np.abs(grads["dbeta"] - fd)) <= 1e-7 * max(1.0, np.max(np.abs(fd)))


def test_one_token_closed_form():
    """One token, zero state, ungated: S_1 = beta k v^T and o = scale beta (q.k) v,
    so dv = beta (scale (q.k) do + dS_T^T k), dq = scale beta (v . do) k and
    dS0 = (I - beta k k^T) (scale q do^T + dS_T)."""
    rng = np.random.default_rng(3)
    dk, dv = 3, 2
    q, k = rng.standard_normal((1, 1, dk)), rng.standard_normal((1, 1, dk))
    v = rng.standard_normal((1, 1, dv))
    b = np.array([[0.4]])
    do, dST = rng.standard_normal((1, 1, dv)), rng.standard_normal((1, 1, dk, dv))
    scale = 0.5
    gr = recurrence_backward(q, k, v, b, None, scale, None, None, do, dST)
    qv, kv, vv, dov, dS = q[0, 0], k[0, 0], v[0, 0], do[0, 0], dST[0, 0]
    assert np.allclose(gr["dv"][0, 0], 0.4 * (scale * (qv @ kv) * dov + dS.T @ kv))
    assert np.allclose(gr["dq"][0, 0], scale * 0.4 * (vv @ dov) * kv)
    M = np.eye(dk) - 0.4 * np.outer(kv, kv)
    assert np.allclose(gr["dS0"][0, 0], M @ (scale * np.outer(qv, dov) + dS))


# ------------------------------------------------------------ planted mistakes
# Each mutation edits one line of a copy of the backward oracle's source (on the
# CPU) and checks that the finite-difference pin fails for some input.
import os  # noqa: E402
import types  # noqa: E402

_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "backward.py")
MUTATIONS = {
    "drop_delta_dk": ("dkk[t, kh] -= bt * (Sd @ du)", "pass"),
    "sign_dq": ("dq[t, kh] += scale * (St @ do[t, h])", "dq[t, kh] -= scale * (St @ do[t, h])"),
    "dq_from_prev_state": ("dq[t, kh] += scale * (St @ do[t, h])", "dq[t, kh] += scale * (Sd @ do[t, h])"),
    "transposed_du": ("du = dS.T @ kt", "du = (dS.T @ kt)[::-1]"),
    "dbeta_from_v_only": ("dbeta[t, h] = du @ (vt - p)", "dbeta[t, h] = du @ vt"),
    "no_decay_carry": ("dS = a * dSd", "dS = dSd"),
    "dg_from_undecayed": ("dg[t, h] = np.sum(dSd * Sd)", "dg[t, h] = np.sum(dSd * S_prev)"),
    "missing_output_inject": ("dS = dS + scale * np.outer(qt, do[t, h])", "dS = dS"),
}


def _mutant(old, new):
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_backward")
    exec(compile(src.replace(old, new), "mutant_backward", "exec"), mod.__dict__)
    return mod.recurrence_backward


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_the_pin(name):
    fn = _mutant(*MUTATIONS[name])
    x, cu, w = problem(5)
    scale = 0.7
    grads = fn(x["q"], x["k"], x["v"], x["beta"], x["g"], scale, x["S0"], cu, w["do"], w["dS_T"])
    worst = 0.0
    for nm, key in NAMES.items():
        fd = finite_difference(x, cu, w, scale, nm)
        worst = max(worst, np.max(np.abs(grads[key] - fd)) / max(1.0, np.max(np.abs(fd))))
    assert worst > 1e-4, (name, worst)
