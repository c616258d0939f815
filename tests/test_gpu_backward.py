"""GPU parity of the backward pass (gdr_chunk_bwd) against the fp64 backward
oracle (``oracle.recurrence_backward``, pinned by finite differences),
element by element, for dq, dk, dv, dbeta, dg and the initial state's
gradient.

The oracle sees exactly the values the GPU sees (inputs and dL/do rounded to
their dtype). Bound: max |x - ref| / rms(ref) <= 1e-4 for fp32 inputs and
2e-2 for bf16 inputs, per gradient (the GPU computes in fp32 either way; the
pages' own tests use 0.006-0.008 on a ratio of rms errors, FLA DeltaNet
article, section 6). Cases: fixed length and variable length (empty,
one-token, one-chunk and ragged sequences), GQA, chunk sizes 16, 32 and 64,
the ungated rule (dg is then the gradient at g = 0), a strongly decaying gate,
every head-dim pair, with and without dL/dS_T, and d_o in fp32. For bf16
inputs at C = 64 with at least 128 (sequence, value head, 16 dv columns)
units, the recompute takes its chunk states from the fp16 chunk pass (cases
bf16_states16_*, the determinism and full-size tests); otherwise from the
five-kernel state pass.
"""
import numpy as np
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth
from gpu_common import TOL, f64, oracle_inputs, rel_err, to_dev
from oracle import recurrence_backward

pytestmark = pytest.mark.gpu


def grads_in(inp, seed, do_f32=False, with_dST=True):
    """dL/do (in o's dtype) and dL/dS_T for an input batch."""
    w = inp["workload"]
    rng = np.random.default_rng(seed)
    B, T = inp["q"].shape[:2]
    do = torch.from_numpy(rng.standard_normal((B, T, w.Nv, w.dv)).astype(np.float32))
    if not do_f32:
        do = do.to(inp["q"].dtype)
    N = inp["N"]
    dST = torch.from_numpy(rng.standard_normal((N, w.Nv, w.dk, w.dv)).astype(np.float32)) if with_dST else None
    return do, dST


def check(label, inp, seed, C=64, do_f32=False, with_dST=True, g_zero_for_oracle=False):
    w = inp["workload"]
    tol = TOL[w.dtype]
    do, dST = grads_in(inp, seed, do_f32, with_dST)
    d = to_dev(inp)
    res = api.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), g=d["g"], scale=inp["scale"],
                        initial_state=d["S0"], d_final_state=None if dST is None else dST.cuda(),
                        cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"], chunk_size=C)
    torch.cuda.synchronize()
    x = oracle_inputs(inp)
    g = x["g"]
    if g is None and g_zero_for_oracle:
        g = np.zeros_like(x["beta"])
    Ttot = x["q"].shape[0]
    ref = recurrence_backward(x["q"], x["k"], x["v"], x["beta"], g, x["scale"], x["S0"], x["cu"],
                              f64(do).reshape(Ttot, w.Nv, w.dv), None if dST is None else f64(dST))
    got = dict(dq=res["dq"], dk=res["dk"], dv=res["dv"], dbeta=res["dbeta"], dg=res["dg"], dS0=res["dh0"])
    errs = {}
    for key, r in ref.items():
        if r is None:
            continue
        xg = f64(got[key]).reshape(r.shape)
        assert np.all(np.isfinite(xg)), (label, key)
        errs[key] = rel_err(xg, r)
    print("%s C=%d %s (tol %.0e)" % (label, C, " ".join("%s %.2e" % kv for kv in errs.items()), tol), flush=True)
    for key, e in errs.items():
        assert e <= tol, (label, key, e)
    return res


CASES = {
    "f32_gqa_T150": dict(B=1, T=150, Nk=1, Nv=2, dk=32, dv=64, dtype="f32", s0="randn"),
    "f32_B2_d128": dict(B=2, T=70, Nk=2, Nv=2, dk=128, dv=128, dtype="f32", s0="randn"),
    "bf16_varlen_gqa": dict(B=1, T=0, Nk=2, Nv=4, dk=64, dv=64, dtype="bf16", s0="randn",
                            lengths=(1, 63, 64, 65, 130, 0)),
    "bf16_T200_d128": dict(B=1, T=200, Nk=1, Nv=1, dk=128, dv=128, dtype="bf16", s0="zero"),
    "bf16_strong_decay": dict(B=1, T=130, Nk=1, Nv=2, dk=64, dv=32, dtype="bf16", g_mean=-2.0, s0="randn"),
    # at least 128 (sequence, value head, 16 dv columns) units: the recompute's
    # chunk states come from the fp16 chunk pass
    "bf16_states16_varlen": dict(B=1, T=0, Nk=2, Nv=8, dk=64, dv=128, dtype="bf16", s0="randn",
                                 lengths=(200, 1, 65, 130)),
    "bf16_states16_B2_d128": dict(B=2, T=150, Nk=4, Nv=8, dk=128, dv=128, dtype="bf16", s0="randn"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_parity(case):
    w = synth.custom(case, **CASES[case])
    check(case, synth.generate(w, seed=400 + len(case)), seed=1)


@pytest.mark.parametrize("C", [16, 32])
def test_backward_chunk_sizes(C):
    w = synth.custom("bwdC", B=1, T=0, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16", s0="randn", lengths=(17, 40, 100))
    check("bwd_C%d" % C, synth.generate(w, seed=420 + C), seed=2, C=C)


def test_backward_f32_chunk16():
    w = synth.custom("bwdC16f", B=1, T=90, Nk=1, Nv=2, dk=32, dv=32, dtype="f32", s0="randn")
    check("bwd_f32_C16", synth.generate(w, seed=431), seed=3, C=16)


def test_backward_ungated_gives_gradient_at_zero_gate():
    w = synth.custom("bwd_ungated", B=1, T=100, Nk=1, Nv=2, dk=64, dv=64, dtype="f32", gated=False, s0="randn")
    check("bwd_ungated", synth.generate(w, seed=432), seed=4, g_zero_for_oracle=True)


def test_backward_without_final_state_gradient_and_fp32_do():
    w = synth.custom("bwd_nodst", B=2, T=80, Nk=1, Nv=2, dk=64, dv=32, dtype="bf16", s0="randn")
    check("bwd_no_dST_f32do", synth.generate(w, seed=433), seed=5, do_f32=True, with_dST=False)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_backward_every_head_dim_pair(dk, dv):
    w = synth.custom("bwd_dims", B=1, T=75, Nk=1, Nv=2, dk=dk, dv=dv, dtype="bf16", s0="randn")
    check("bwd_dims(%d,%d)" % (dk, dv), synth.generate(w, seed=440 + dk + dv), seed=6)


def test_backward_long_sequence_d128():
    """16 chunks of one sequence at dk = dv = 128 with GQA, against the oracle."""
    w = synth.custom("bwd_long", B=1, T=1024, Nk=1, Nv=2, dk=128, dv=128, dtype="bf16", s0="randn", g_mean=6.0)
    check("bwd_long_T1024", synth.generate(w, seed=450), seed=7)


def test_backward_is_deterministic():
    """Two runs on the same inputs give the same bits for every gradient."""
    w = synth.custom("bwd_det", B=1, T=0, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16", s0="randn",
                     lengths=(700, 1, 64, 333))
    inp = synth.generate(w, seed=460)
    do, dST = grads_in(inp, 8)
    d = to_dev(inp)
    runs = []
    for _ in range(2):
        runs.append(api.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), g=d["g"], scale=inp["scale"],
                                  initial_state=d["S0"], d_final_state=dST.cuda(), cu_seqlens=d["cu_seqlens"],
                                  cu_seqlens_cpu=inp["cu_seqlens"]))
        torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.equal(runs[0][key], runs[1][key]), key


def test_backward_full_size_linearity():
    """The long-context workload at full size (T = 65536, Nk = 16, Nv = 32,
    dk = dv = 128, bf16) in the configuration the benchmark times. The oracle
    cannot run at this size, so properties that hold at any size are checked:
    every gradient is finite; the backward is linear in (dL/do, dL/dS_T), so
    doubling both doubles every gradient exactly (scaling by 2 is exact in
    floating point, also for the hi + lo bf16 split of the reverse state
    pass's operands, and every sum runs in a fixed order, with no atomics); the
    gradients of a sum are the sum of the gradients to within 1e-3 of the rms
    (the state pass keeps about 16 bits of dS, W^T and Z per product, and its
    rounding differs between the three runs and accumulates over the 1,024
    reverse chunk steps: measured 1.4e-4 on dk, 3.5e-6 on dq)."""
    w = synth.WORKLOADS[5]
    inp = synth.generate(w, seed=5)
    d = to_dev(inp)
    rng = np.random.default_rng(12)
    B, T = inp["q"].shape[:2]
    do1 = torch.from_numpy(rng.standard_normal((B, T, w.Nv, w.dv)).astype(np.float32)).cuda()
    do2 = torch.from_numpy(rng.standard_normal((B, T, w.Nv, w.dv)).astype(np.float32)).cuda()
    dS1 = torch.from_numpy(rng.standard_normal((1, w.Nv, w.dk, w.dv)).astype(np.float32)).cuda()
    dS2 = torch.from_numpy(rng.standard_normal((1, w.Nv, w.dk, w.dv)).astype(np.float32)).cuda()

    def run(do, dS):
        res = api.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do, g=d["g"], scale=inp["scale"],
                            initial_state=d["S0"], d_final_state=dS)
        torch.cuda.synchronize()
        return res

    r1 = run(do1, dS1)
    r1x2 = run(2 * do1, 2 * dS1)
    r2 = run(do2, dS2)
    r12 = run(do1 + do2, dS1 + dS2)
    for key in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        a = r1[key]
        assert bool(torch.isfinite(a).all()), key
        assert torch.equal(r1x2[key], 2 * a), key
        ref = (a.double() + r2[key].double())
        err = float((r12[key].double() - ref).abs().max() / ref.pow(2).mean().sqrt())
        print("full-size %s: additivity max|d|/rms %.2e" % (key, err), flush=True)
        assert err < 1e-3, (key, err)
