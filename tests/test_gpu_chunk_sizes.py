"""GPU parity at chunk sizes C = 16 and 32 (five-kernel path) against the
fp64 oracle, element by element, and agreement across C = 16, 32, 64.

The chunk size changes only the order of the arithmetic: the exact result is
the token recurrence for every C. Cases put sequence ends on, just before and
just after chunk boundaries, and cover GQA, the ungated rule, fp32 and bf16,
every head-dim pair at one C, an initial state, and segment-parallel state
passing at C = 32.
"""
import numpy as np
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth
from gpu_common import TOL, bf16_rounding_excess, f64, oracle_inputs, rel_err, run_gpu, to_dev
from oracle import recurrence

pytestmark = pytest.mark.gpu


def oracle_ref(inp):
    x = oracle_inputs(inp)
    return recurrence(x["q"], x["k"], x["v"], x["beta"], x["g"], x["scale"], x["S0"], x["cu"])


def check(label, inp, C, ref=None):
    w = inp["workload"]
    tol = TOL[w.dtype]
    o_ref, S_ref = oracle_ref(inp) if ref is None else ref
    o, S = run_gpu(inp, out_f32=True, chunk_size=C)
    eo = rel_err(f64(o).reshape(o_ref.shape), o_ref)
    es = rel_err(f64(S), S_ref)
    msg = "%s C=%d err o %.3e S_T %.3e (tol %.0e)" % (label, C, eo, es, tol)
    if w.dtype == "bf16":
        ob, _ = run_gpu(inp, chunk_size=C)
        exc = bf16_rounding_excess(f64(ob).reshape(o_ref.shape), o_ref)
        msg += " | bf16-out excess over rne(exact) %.3e" % exc
        assert exc <= TOL["bf16"]
    print(msg, flush=True)
    assert np.all(np.isfinite(f64(o))) and np.all(np.isfinite(f64(S)))
    assert eo <= tol and es <= tol
    return o, S


CASES = {
    "bf16_B2_T150": dict(B=2, T=150, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16", s0="randn"),
    "bf16_varlen_edges": dict(B=1, T=0, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16", s0="randn",
                              lengths=(1, 15, 16, 17, 31, 32, 33, 0, 64, 100)),
    "bf16_ungated": dict(B=1, T=97, Nk=1, Nv=1, dk=32, dv=128, dtype="bf16", gated=False, s0="zero"),
    "bf16_strong_decay": dict(B=1, T=200, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16", g_mean=-2.0),
    "f32_T130": dict(B=1, T=130, Nk=2, Nv=2, dk=64, dv=32, dtype="f32", s0="randn"),
    "f32_varlen": dict(B=1, T=0, Nk=1, Nv=2, dk=128, dv=64, dtype="f32", lengths=(17, 0, 48, 5)),
}


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("case", sorted(CASES))
def test_chunk_size_parity(case, C):
    w = synth.custom(case, **CASES[case])
    inp = synth.generate(w, seed=200 + len(case))
    check(case, inp, C)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_every_head_dim_pair_C32_bf16(dk, dv):
    w = synth.custom("dims32_%d_%d" % (dk, dv), B=1, T=100, Nk=1, Nv=2, dk=dk, dv=dv, dtype="bf16", s0="randn")
    check("dims(%d,%d)" % (dk, dv), synth.generate(w, seed=dk * 3 + dv), 32)


def test_chunk_sizes_agree():
    """C = 16, 32 and 64 give the same result (config 2): C = 16 and 32 run the
    five kernels at fp32-level accuracy and agree to fp32 rounding; C = 64 runs
    the production path with fp16 operands and agrees to a few 1e-3 of rms."""
    inp = synth.generate(synth.WORKLOADS[2], seed=2)
    outs = {C: run_gpu(inp, out_f32=True, chunk_size=C) for C in (16, 32, 64)}
    eo = rel_err(f64(outs[16][0]), f64(outs[32][0]))
    es = rel_err(f64(outs[16][1]), f64(outs[32][1]))
    print("C=16 vs C=32: o %.2e S_T %.2e" % (eo, es), flush=True)
    assert eo < 1e-4 and es < 1e-4
    for C in (16, 32):
        eo = rel_err(f64(outs[C][0]), f64(outs[64][0]))
        es = rel_err(f64(outs[C][1]), f64(outs[64][1]))
        print("C=%d vs C=64: o %.2e S_T %.2e" % (C, eo, es), flush=True)
        assert eo < 1e-2 and es < 1e-2


def test_segmented_at_chunk_size_32():
    w = synth.custom("seg32", B=1, T=32 * 23 + 7, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16", s0="randn")
    inp = synth.generate(w, seed=301)
    d = to_dev(inp)
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                         out_dtype=torch.float32, chunk_size=32, segment_chunks=5)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_ref(inp)
    eo, es = rel_err(f64(o).reshape(o_ref.shape), o_ref), rel_err(f64(S), S_ref)
    print("segmented C=32: err o %.3e S_T %.3e" % (eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
