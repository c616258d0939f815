"""Backward pass of the gated delta rule, token by token, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reverse-mode differentiation of the token recurrence that ``recurrence``
computes. This is backpropagation through time: the state gradient gathers the
output's contribution at every step and is carried to the previous step
through the step's decay (FLA notes page, "fused recurrent bwd": the total
state gradient at step t is q_t do_t^T plus the decayed gradient from step
t + 1). The delta rule adds the error-correction term. The gradients the
pages' tests compare are dq, dk, dv, dbeta and dh0 (FLA DeltaNet article,
section 6); dg, the gate's gradient, completes the gated form.

Forward step t of sequence n and value head h (q/k head kh = h / (Nv / Nk);
ChunkGatedDeltaRule page, section 1; the delta is read from the decayed
state):

    a  = exp(g_t)
    Sd = a S_{t-1}                     decayed state
    p  = Sd^T k_t                      prediction of v_t
    u  = beta_t (v_t - p)
    S_t = Sd + k_t u^T
    o_t = scale S_t^T q_t

Reverse step, with dS the gradient of the loss with respect to S_t (from
later steps, or dS_T at the last token):

    dS   += scale q_t do_t^T
    dq_t += scale S_t do_t
    du    = dS^T k_t;      dk_t += dS u
    dbeta_t = du . (v_t - p);   dv_t = beta_t du
    dSd   = dS - beta_t k_t du^T;   dk_t -= beta_t Sd du
    dg_t  = sum(dSd (.) Sd)    (since dSd/dg = d(a S_{t-1})/dg = Sd)
    dS    = a dSd              gradient with respect to S_{t-1}

dq and dk sum over the value heads that share a q/k head. After a sequence's
first token, dS is the gradient with respect to its initial state.

Pinned by ``tests/test_oracle_backward.py``: central finite differences of
the fp64 forward (``recurrence``) for every input, on small problems with
GQA, variable lengths, an empty sequence, the ungated rule and an initial
state.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def recurrence_backward(q, k, v, beta, g=None, scale=None, S0=None, cu_seqlens=None, do=None,
                        dS_T=None) -> dict:
    """Gradients of L = sum(do * o) + sum(dS_T * S_T) for the token recurrence.

    q, k: [Ttot, Nk, dk]; v: [Ttot, Nv, dv]; beta, g: [Ttot, Nv] (g None:
    ungated); S0: [N, Nv, dk, dv] or None (zeros); cu_seqlens: [N + 1]
    offsets, or None for one sequence; do: [Ttot, Nv, dv]; dS_T: [N, Nv, dk,
    dv] or None (zeros).
    Returns dict dq [Ttot, Nk, dk], dk, dv [Ttot, Nv, dv], dbeta [Ttot, Nv],
    dg [Ttot, Nv] (None when g is None), dS0 [N, Nv, dk, dv].
    """
    f = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, beta, g, S0, do, dS_T = map(f, (q, k, v, beta, g, S0, do, dS_T))
    Ttot, Nk, dk = q.shape
    Nv, dv = v.shape[1:]
    cu = np.array([0, Ttot], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    group = Nv // Nk
    if scale is None:
        scale = dk ** -0.5

    dq = np.zeros((Ttot, Nk, dk))
    dkk = np.zeros((Ttot, Nk, dk))
    dvv = np.zeros((Ttot, Nv, dv))
    dbeta = np.zeros((Ttot, Nv))
    dg = np.zeros((Ttot, Nv))
    dS0 = np.zeros((N, Nv, dk, dv))

    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(Nv):
            kh = h // group
            # forward, keeping the state entering every token
            S = S0[n, h].copy() if S0 is not None else np.zeros((dk, dv))
            prev = []
            for t in range(s, e):
                prev.append(S)
                a = np.exp(g[t, h]) if g is not None else 1.0
                Sd = a * S
                u = beta[t, h] * (v[t, h] - Sd.T @ k[t, kh])
                S = Sd + np.outer(k[t, kh], u)
            # reverse
            dS = dS_T[n, h].copy() if dS_T is not None else np.zeros((dk, dv))
            for t in range(e - 1, s - 1, -1):
                S_prev = prev[t - s]
                a = np.exp(g[t, h]) if g is not None else 1.0
                kt, qt, vt, bt = k[t, kh], q[t, kh], v[t, h], beta[t, h]
                Sd = a * S_prev
                p = Sd.T @ kt
                u = bt * (vt - p)
                St = Sd + np.outer(kt, u)
                dS = dS + scale * np.outer(qt, do[t, h])
                dq[t, kh] += scale * (St @ do[t, h])
                du = dS.T @ kt
                dkk[t, kh] += dS @ u
                dbeta[t, h] = du @ (vt - p)
                dvv[t, h] = bt * du
                dSd = dS - bt * np.outer(kt, du)
                dkk[t, kh] -= bt * (Sd @ du)
                dg[t, h] = np.sum(dSd * Sd)
                dS = a * dSd
            dS0[n, h] = dS
    return dict(dq=dq, dk=dkk, dv=dvv, dbeta=dbeta, dg=dg if g is not None else None, dS0=dS0)
