"""Seeded synthetic workloads for the chunked gated delta-rule forward.

This module only draws inputs. It holds none of the method's arithmetic, so
the CPU oracle and the HIP path can both consume its output without sharing
any computation.

Value recipe (shared by every workload, following the usage example of the
FLA DeltaNet article, section 5 "API", and the gated operator's input table on
the ChunkGatedDeltaRule page, section 1):

* q, k: standard normal, L2-normalised per (token, head) over dk in fp32,
  then stored in the io dtype (bf16 rounding is round-to-nearest-even).
* v: standard normal, stored in the io dtype.
* beta: sigmoid of a standard normal, stored in the io dtype.
* g: logsigmoid(mu + standard normal) in fp32, so every g is <= 0 (log-domain
  forget gate); absent for the ungated workload.
* S0: 0.1 * standard normal in fp32 ("N(0, 0.1)" read as a standard
  deviation), or absent (zeros).
* Variable-length batches: lengths drawn uniformly from [lo, hi], packed
  along one token axis (B = 1) with cumulative offsets ``cu_seqlens``.

Draw order from ``numpy.random.default_rng(seed)`` is fixed: lengths (varlen
only), q, k, v, beta logits, g logits, S0. All draws are fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # batch rows (1 when varlen)
    T: int                 # tokens per batch row (ignored when varlen)
    Nk: int                # q/k heads
    Nv: int                # v heads (multiple of Nk)
    dk: int
    dv: int
    dtype: str             # "bf16" or "f32" (q, k, v, beta, o)
    gated: bool = True
    g_mean: float = 4.0    # mu in g = logsigmoid(mu + N(0,1))
    s0: str = "randn"      # "randn" (0.1 * N(0,1)) or "zero" (absent)
    varlen: Optional[tuple] = None   # (num_seqs, lo, hi): lengths drawn uniformly in [lo, hi]
    lengths: Optional[tuple] = None  # explicit packed sequence lengths (varlen, B = 1)
    scale: Optional[float] = None    # None -> dk ** -0.5

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads used for parity and measurement.
WORKLOADS = {
    1: Workload("ungated-f32-H2-T256-d32", B=1, T=256, Nk=2, Nv=2, dk=32, dv=32,
                dtype="f32", gated=False, s0="zero"),
    2: Workload("gated-bf16-B2-H4-T1000-d64", B=2, T=1000, Nk=4, Nv=4, dk=64, dv=64,
                dtype="bf16", g_mean=4.0, s0="randn"),
    3: Workload("gated-bf16-B4-H16-T4096-d128", B=4, T=4096, Nk=16, Nv=16, dk=128, dv=128,
                dtype="bf16", g_mean=4.0, s0="zero"),
    4: Workload("gqa-varlen-bf16-Nk16-Nv32-64seq-d128", B=1, T=0, Nk=16, Nv=32, dk=128, dv=128,
                dtype="bf16", g_mean=4.0, s0="randn", varlen=(64, 1, 8192)),
    5: Workload("gqa-bf16-Nk16-Nv32-T65536-d128", B=1, T=65536, Nk=16, Nv=32, dk=128, dv=128,
                dtype="bf16", g_mean=6.0, s0="zero"),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2norm_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    # log(sigmoid(x)) = -log1p(exp(-x)), written stably for both signs.
    out = np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))
    return out.astype(np.float32)


def seq_lengths(w: Workload, rng: np.random.Generator) -> Optional[np.ndarray]:
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int64)
    if w.varlen is None:
        return None
    n, lo, hi = w.varlen
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def generate(w: Workload, seed: int) -> dict:
    """Draw one batch for workload ``w``. Returns CPU torch tensors.

    Keys: q [B,T,Nk,dk], k [B,T,Nk,dk], v [B,T,Nv,dv], beta [B,T,Nv] (io dtype),
    g [B,T,Nv] fp32 or None, S0 [N,Nv,dk,dv] fp32 or None, cu_seqlens int64 [N+1]
    or None, scale (float), N (number of sequences), workload.
    """
    rng = np.random.default_rng(seed)
    lengths = seq_lengths(w, rng)
    if lengths is not None:
        B, T = 1, int(lengths.sum())
        N = len(lengths)
        cu = np.zeros(N + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
    else:
        B, T, N, cu = w.B, w.T, w.B, None
    tdt = _TORCH_DTYPE[w.dtype]

    q = _l2norm_last(_normal(rng, (B, T, w.Nk, w.dk)))
    k = _l2norm_last(_normal(rng, (B, T, w.Nk, w.dk)))
    v = _normal(rng, (B, T, w.Nv, w.dv))
    beta = _sigmoid(_normal(rng, (B, T, w.Nv)))
    g = _logsigmoid(np.float32(w.g_mean) + _normal(rng, (B, T, w.Nv))) if w.gated else None
    S0 = (np.float32(0.1) * _normal(rng, (N, w.Nv, w.dk, w.dv))) if w.s0 == "randn" else None

    out = dict(
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        beta=torch.from_numpy(beta).to(tdt),
        g=None if g is None else torch.from_numpy(g),
        S0=None if S0 is None else torch.from_numpy(S0),
        cu_seqlens=None if cu is None else torch.from_numpy(cu),
        scale=float(w.scale if w.scale is not None else w.dk ** -0.5),
        N=N,
        workload=w,
    )
    return out


def custom(name="custom", **kw) -> Workload:
    """Small ad-hoc workload for tests (same value recipe)."""
    base = dict(B=1, T=128, Nk=1, Nv=1, dk=32, dv=32, dtype="f32")
    base.update(kw)
    return Workload(name, **base)
