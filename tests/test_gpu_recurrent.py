"""GPU parity of the token-by-token (fused recurrent) forward against the fp64
oracle, element by element: decode steps from a given state, short and
variable-length inputs, GQA, all head dims, fp32 and bf16 inputs, the in-kernel
L2 normalisation of q and k, and agreement with the chunked path."""
import numpy as np
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth
from gpu_common import TOL, f64, oracle_inputs, rel_err, to_dev, bf16_rounding_excess
from oracle import l2_normalize, recurrence

pytestmark = pytest.mark.gpu


def run_rec(inp, l2norm=False, out_f32=True, output_final_state=True):
    d = to_dev(inp)
    o, S = api.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"],
                             initial_state=d["S0"], output_final_state=output_final_state,
                             cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"],
                             use_qk_l2norm_in_kernel=l2norm, out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    return o, S


def oracle_ref(inp, l2norm=False):
    x = oracle_inputs(inp)
    q, k = x["q"], x["k"]
    if l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    return recurrence(q, k, x["v"], x["beta"], x["g"], x["scale"], x["S0"], x["cu"])


def check(name, inp, l2norm=False):
    w = inp["workload"]
    tol = TOL[w.dtype]
    o, S = run_rec(inp, l2norm=l2norm)
    o_ref, S_ref = oracle_ref(inp, l2norm)
    eo = rel_err(f64(o).reshape(o_ref.shape), o_ref)
    es = rel_err(f64(S), S_ref)
    ob, _ = run_rec(inp, l2norm=l2norm, out_f32=False, output_final_state=False)
    exc = bf16_rounding_excess(f64(ob).reshape(o_ref.shape), o_ref) if w.dtype == "bf16" else None
    print("%s recurrent fp32-out err o %.3e  S_T %.3e (tol %.0e)%s" % (
        name, eo, es, tol, "" if exc is None else " | io-dtype out: excess over rne(exact) %.3e" % exc))
    assert eo <= tol and es <= tol
    assert exc is None or exc <= tol
    return o, S


def decode(Nseq, Nk, Nv, dk, dv, dtype, seed):
    """Nseq sequences of one token each, from a random state (a decode step)."""
    w = synth.custom("decode", B=1, T=0, Nk=Nk, Nv=Nv, dk=dk, dv=dv, dtype=dtype, s0="randn",
                     lengths=tuple([1] * Nseq))
    return synth.generate(w, seed=seed)


CASES = {
    "decode_bf16_gqa": lambda: decode(8, 2, 4, 128, 128, "bf16", 21),
    "decode_f32_d64": lambda: decode(5, 2, 2, 64, 64, "f32", 22),
    "short_T64_bf16": lambda: synth.generate(synth.custom("short", B=2, T=64, Nk=2, Nv=4, dk=128, dv=128,
                                                          dtype="bf16", s0="randn"), seed=23),
    "short_T33_f32_ungated": lambda: synth.generate(synth.custom("short_ungated", B=2, T=33, Nk=2, Nv=2,
                                                                 dk=32, dv=32, dtype="f32", gated=False,
                                                                 s0="zero"), seed=24),
    "varlen_bf16": lambda: synth.generate(synth.custom("varlen", B=1, T=0, Nk=2, Nv=4, dk=64, dv=128,
                                                       dtype="bf16", s0="randn", lengths=(1, 17, 0, 40, 64)),
                                          seed=25),
    "dv32_dk128_f32": lambda: synth.generate(synth.custom("dv32", B=1, T=50, Nk=1, Nv=2, dk=128, dv=32,
                                                          dtype="f32", s0="randn"), seed=26),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_recurrent_parity(case):
    check(case, CASES[case]())


@pytest.mark.parametrize("case", ["decode_bf16_gqa", "short_T64_bf16", "varlen_bf16"])
def test_recurrent_qk_l2norm(case):
    """With the flag, the kernel normalises q and k itself: the result matches the
    oracle run on normalised q, k, and differs from the unnormalised run."""
    inp = CASES[case]()
    # scale q, k away from unit length so that the normalisation matters
    inp["q"] = (inp["q"].float() * 3.0).to(inp["q"].dtype)
    inp["k"] = (inp["k"].float() * 0.5).to(inp["k"].dtype)
    o, _ = check(case + "+l2norm", inp, l2norm=True)
    o_plain, _ = run_rec(inp, l2norm=False)
    assert rel_err(f64(o_plain), f64(o)) > 1e-2


@pytest.mark.parametrize("cfg", [2, 3])
def test_recurrent_matches_chunked_path(cfg):
    """Both paths compute the same forward: compare them directly on a config
    (the chunked production path rounds its derived operands to fp16, the
    token-by-token path works in fp32: they agree to a few 1e-3 of rms)."""
    w = synth.WORKLOADS[cfg]
    inp = synth.generate(w, seed=cfg)
    o_r, S_r = run_rec(inp)
    d = to_dev(inp)
    o_c, S_c = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                             cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    eo, es = rel_err(f64(o_r), f64(o_c)), rel_err(f64(S_r), f64(S_c))
    print("cfg%d recurrent vs chunked: o %.2e S_T %.2e" % (cfg, eo, es))
    assert eo < 1e-2 and es < 1e-2


def test_recurrent_decode_continues_a_sequence():
    """Prefix by the chunked path, then token-by-token decode steps from its final
    state, equal the oracle over the whole sequence."""
    w = synth.custom("prefix_decode", B=1, T=70, Nk=2, Nv=4, dk=64, dv=64, dtype="bf16", s0="randn")
    inp = synth.generate(w, seed=27)
    d = to_dev(inp)
    T0 = 66
    o1, S1 = api.chunk_fwd(d["q"][:, :T0].contiguous(), d["k"][:, :T0].contiguous(), d["v"][:, :T0].contiguous(),
                           d["beta"][:, :T0].contiguous(), g=d["g"][:, :T0].contiguous(), scale=inp["scale"],
                           initial_state=d["S0"], out_dtype=torch.float32)
    S = S1
    outs = [o1]
    for t in range(T0, 70):
        sl = lambda x: x[:, t:t + 1].contiguous()
        o_t, S = api.recurrent_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), g=sl(d["g"]),
                                   scale=inp["scale"], initial_state=S, out_dtype=torch.float32)
        outs.append(o_t)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    o_ref, S_ref = oracle_ref(inp)
    eo, es = rel_err(f64(o).reshape(o_ref.shape), o_ref), rel_err(f64(S), S_ref)
    print("prefix (chunked) + 4 decode steps (recurrent): o %.2e S_T %.2e" % (eo, es))
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_recurrent_empty_and_no_final_state():
    inp = CASES["varlen_bf16"]()
    o, S = run_rec(inp, output_final_state=False)
    assert S is None
    o_ref, _ = oracle_ref(inp)
    assert rel_err(f64(o).reshape(o_ref.shape), o_ref) <= TOL["bf16"]
