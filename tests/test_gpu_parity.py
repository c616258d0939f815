"""GPU parity: the HIP path against the fp64 oracle, element by element.

Error metric: max |x - ref| / rms(ref) per tensor; bounds 2e-2 for bf16 inputs
and 1e-4 for fp32 inputs (fp32 accumulation in both). Inputs are the seeded
synthetic workloads of chunkwise_gated_delta_local_amd.synth; the oracle sees
exactly the rounded values the GPU sees.
"""
import numpy as np
import pytest
import torch

import frag_layout as fl
from gpu_common import TOL, bf16_rounding_excess, oracle_inputs, rel_err, run_gpu
from oracle import chunked_forward, recurrence
from chunkwise_gated_delta_local_amd import synth

pytestmark = pytest.mark.gpu


def oracle_reference(inp, heads=None):
    """Token recurrence (fp64) for all value heads, or for a sample of them
    (every sequence); the sampled run pairs each value head with its own q/k
    head. Returns (o_ref [Ttot, H, dv], S_ref [N, H, dk, dv], heads)."""
    w = inp["workload"]
    sub = dict(inp)
    if heads is not None:
        heads = list(heads)
        kheads = [h // (w.Nv // w.Nk) for h in heads]
        sub.update(q=inp["q"][:, :, kheads], k=inp["k"][:, :, kheads], v=inp["v"][:, :, heads],
                   beta=inp["beta"][:, :, heads], g=None if inp["g"] is None else inp["g"][:, :, heads],
                   S0=None if inp["S0"] is None else inp["S0"][:, heads])
    x = oracle_inputs(sub)
    o_ref, S_ref = recurrence(x["q"], x["k"], x["v"], x["beta"], x["g"], x["scale"], x["S0"], x["cu"])
    return o_ref, S_ref, heads


def to_np(t, heads, shape):
    if heads is not None:
        t = t[:, :, heads] if t.dim() == 4 and t.shape[0] != shape[0] else t[:, heads]
    return t.detach().cpu().double().numpy().reshape(shape)


def check_run(inp, ref, tol, label, beta_f32=False):
    """fp32 output: the max|d|/rms bound. bf16 inputs also run with bf16
    output, whose excess over the correctly rounded exact value's own error
    (bf16_rounding_excess) must stay within the same bound."""
    o_ref, S_ref, heads = ref
    o32, S = run_gpu(inp, beta_f32=beta_f32, out_f32=True)
    o = to_np(o32[:, :, heads] if heads is not None else o32, None, o_ref.shape)
    Sn = to_np(S[:, heads] if heads is not None else S, None, S_ref.shape)
    eo, es = rel_err(o, o_ref), rel_err(Sn, S_ref)
    msg = "%s fp32-out err o %.3e  S_T %.3e (tol %.0e)" % (label, eo, es, tol)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sn)), label
    if inp["workload"].dtype == "bf16":
        o16, S16 = run_gpu(inp, beta_f32=beta_f32)
        assert torch.equal(S16, S), (label, "final state depends on the output dtype")
        ob = to_np(o16[:, :, heads] if heads is not None else o16, None, o_ref.shape)
        excess = bf16_rounding_excess(ob, o_ref)
        msg += " | bf16-out err o %.3e, excess over rne(exact) %.3e" % (rel_err(ob, o_ref), excess)
        assert excess <= tol, (label, "bf16 output", excess)
    print(msg, flush=True)
    assert eo <= tol, (label, "o", eo)
    assert es <= tol, (label, "S_T", es)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_full_parity(cfg):
    w = synth.WORKLOADS[cfg]
    inp = synth.generate(w, seed=cfg)
    check_run(inp, oracle_reference(inp), TOL[w.dtype], "cfg%d" % cfg)


@pytest.mark.parametrize("cfg", [4, 5])
def test_config_full_size_all_heads(cfg):
    """Full-size workloads in the bench's launch configuration, every value
    head compared with the token recurrence. The GPU runs once over all heads;
    the oracle runs per group of eight value heads (with their q/k heads) so
    that its fp64 copies stay a few GB."""
    w = synth.WORKLOADS[cfg]
    inp = synth.generate(w, seed=cfg)
    tol = TOL[w.dtype]
    o32, S = run_gpu(inp, out_f32=True)
    o16, S16 = run_gpu(inp)
    assert torch.equal(S16, S), ("cfg%d" % cfg, "final state depends on the output dtype")
    Ttot = o32.shape[0] * o32.shape[1]
    o32 = o32.reshape(Ttot, w.Nv, w.dv)
    o16 = o16.reshape(Ttot, w.Nv, w.dv)
    eo = es = ex = 0.0
    group = 8
    for h0 in range(0, w.Nv, group):
        heads = list(range(h0, min(w.Nv, h0 + group)))
        o_ref, S_ref, _ = oracle_reference(inp, heads)
        o_ref = o_ref.reshape(Ttot, len(heads), w.dv)
        o = o32[:, h0:h0 + len(heads)].double().cpu().numpy()
        ob = o16[:, h0:h0 + len(heads)].double().cpu().numpy()
        Sn = S[:, h0:h0 + len(heads)].double().cpu().numpy().reshape(S_ref.shape)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sn))
        eo, es = max(eo, rel_err(o, o_ref)), max(es, rel_err(Sn, S_ref))
        ex = max(ex, bf16_rounding_excess(ob, o_ref))
        print("cfg%d heads %d..%d: o %.3e S_T %.3e bf16 excess %.3e" % (cfg, heads[0], heads[-1], eo, es, ex),
              flush=True)
    assert eo <= tol and es <= tol and ex <= tol, (cfg, eo, es, ex)


EDGE = [
    # name, workload kwargs
    ("T1", dict(B=2, T=1, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16")),
    ("T63", dict(B=2, T=63, Nk=2, Nv=2, dk=64, dv=32, dtype="bf16")),
    ("T64", dict(B=1, T=64, Nk=1, Nv=4, dk=32, dv=128, dtype="bf16")),
    ("T65", dict(B=3, T=65, Nk=2, Nv=8, dk=128, dv=64, dtype="bf16")),
    ("f32_d64", dict(B=1, T=200, Nk=2, Nv=4, dk=64, dv=64, dtype="f32")),
    ("f32_d128_ungated", dict(B=1, T=130, Nk=1, Nv=1, dk=128, dv=128, dtype="f32", gated=False)),
    ("varlen_zero_len", dict(B=1, T=0, Nk=2, Nv=4, dk=64, dv=64, dtype="bf16", lengths=(0, 5, 0, 64, 129, 1))),
    ("gqa4", dict(B=1, T=300, Nk=1, Nv=4, dk=128, dv=128, dtype="bf16")),
    ("near_one_decay", dict(B=1, T=1000, Nk=1, Nv=2, dk=128, dv=128, dtype="bf16", g_mean=6.0, s0="zero")),
    ("strong_decay", dict(B=1, T=256, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16", g_mean=-2.0)),
]


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_every_head_dim_pair_bf16(dk, dv):
    """Every (dk, dv) instantiation of the fused path: several chunks, a tail,
    GQA, an initial state."""
    w = synth.custom("dims_%d_%d" % (dk, dv), B=2, T=150, Nk=1, Nv=2, dk=dk, dv=dv, dtype="bf16", s0="randn")
    inp = synth.generate(w, seed=dk + dv)
    check_run(inp, oracle_reference(inp), TOL["bf16"], "dims(%d,%d)" % (dk, dv))


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, kw):
    w = synth.custom(name, **kw)
    inp = synth.generate(w, seed=100 + len(name))
    check_run(inp, oracle_reference(inp), TOL[w.dtype], name)


def test_beta_f32_with_bf16_io():
    w = synth.custom("beta32", B=1, T=150, Nk=2, Nv=2, dk=64, dv=64, dtype="bf16")
    inp = synth.generate(w, seed=7)
    check_run(inp, oracle_reference(inp), TOL["bf16"], "beta_f32", beta_f32=True)


def test_absent_gate_equals_zero_gate_bitwise():
    w = synth.custom("g0", B=1, T=200, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16")
    inp = synth.generate(w, seed=8)
    inp_zero = dict(inp, g=torch.zeros_like(inp["g"]))
    inp_none = dict(inp, g=None)
    o1, S1 = run_gpu(inp_zero)
    o2, S2 = run_gpu(inp_none)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_absent_state_equals_zero_state_bitwise():
    w = synth.custom("s0", B=2, T=100, Nk=1, Nv=2, dk=64, dv=64, dtype="bf16")
    inp = synth.generate(w, seed=9)
    o1, S1 = run_gpu(dict(inp, S0=torch.zeros_like(inp["S0"])))
    o2, S2 = run_gpu(dict(inp, S0=None))
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_deterministic_bitwise():
    w = synth.custom("det", B=1, T=500, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16")
    inp = synth.generate(w, seed=10)
    o1, S1 = run_gpu(inp)
    o2, S2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_no_final_state_requested():
    w = synth.custom("nofs", B=1, T=100, Nk=1, Nv=1, dk=64, dv=64, dtype="bf16")
    inp = synth.generate(w, seed=11)
    o, S = run_gpu(inp, output_final_state=False)
    assert S is None
    o2, S2 = run_gpu(inp)
    assert torch.equal(o, o2)


def test_empty_sequence_batch_returns_initial_state():
    w = synth.custom("empty", B=1, T=0, Nk=1, Nv=2, dk=32, dv=32, dtype="bf16", lengths=(0, 0))
    inp = synth.generate(w, seed=12)
    o, S = run_gpu(inp)
    assert o.numel() == 0
    assert torch.equal(S.cpu(), inp["S0"])


# ------------------------------------------------------------ per-kernel parity
KERNEL_CASES = [
    ("cfg2", synth.WORKLOADS[2], 2, 64),
    ("gqa_varlen", synth.custom("gqa_varlen", B=1, T=0, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16",
                                lengths=(1, 63, 64, 65, 130)), 21, 64),
    ("f32", synth.custom("f32k", B=1, T=150, Nk=1, Nv=2, dk=32, dv=64, dtype="f32"), 22, 64),
    ("gqa_varlen_C32", synth.custom("gqa_varlen32", B=1, T=0, Nk=2, Nv=4, dk=128, dv=64, dtype="bf16",
                                    lengths=(1, 31, 32, 33, 100)), 23, 32),
    ("gqa_varlen_C16", synth.custom("gqa_varlen16", B=1, T=0, Nk=2, Nv=4, dk=64, dv=128, dtype="bf16",
                                    lengths=(1, 15, 16, 17, 70)), 24, 16),
    ("f32_C16", synth.custom("f32k16", B=1, T=75, Nk=1, Nv=2, dk=32, dv=64, dtype="f32"), 25, 16),
    ("f32_C32", synth.custom("f32k32", B=2, T=70, Nk=1, Nv=1, dk=64, dv=32, dtype="f32"), 26, 32),
]


@pytest.mark.parametrize("name,w,seed,C", KERNEL_CASES, ids=[c[0] for c in KERNEL_CASES])
def test_intermediates_match_chunked_oracle(name, w, seed, C):
    """Each of the five kernels against the chunked oracle's intermediate at
    chunk size C: K1 -> G, K2 -> A, K3 -> W, U (and K^T), K4 -> H, V_new, S_T,
    K5 -> o."""
    inp = synth.generate(w, seed=seed)
    res = run_gpu(inp, debug=True, out_f32=True, chunk_size=C)
    x = oracle_inputs(inp)
    ref = chunked_forward(x["q"], x["k"], x["v"], x["beta"], x["g"], x["scale"], x["S0"], x["cu"],
                          chunk_size=C, intermediates=True)
    chunks = ref["chunks"]
    Ttot = x["q"].shape[0]
    tol = TOL[w.dtype]
    assert res["num_chunks"] == len(chunks)
    cpu = lambda t: t.detach().cpu().double().numpy()
    errs = {}
    errs["G"] = rel_err(cpu(res["G"]), ref["G"]) if w.gated else float(np.max(np.abs(cpu(res["G"]))))
    errs["A"] = rel_err(cpu(res["A"]), ref["A"])
    W = fl.W_natural(cpu(res["W"]))
    U = fl.U_natural(cpu(res["U"]))
    VN = fl.VN_natural(cpu(res["VN"]))
    K = fl.KT_natural(cpu(res["KT"]))
    assert fl.pad_rows_are_zero(W, chunks) and fl.pad_rows_are_zero(U, chunks)
    assert fl.pad_rows_are_zero(VN, chunks) and fl.pad_rows_are_zero(K, chunks)
    errs["W"] = rel_err(fl.chunk_rows_to_tokens(W, chunks, Ttot), ref["W"])
    errs["U"] = rel_err(fl.chunk_rows_to_tokens(U, chunks, Ttot), ref["U"])
    errs["K"] = rel_err(fl.chunk_rows_to_tokens(K, chunks, Ttot), x["k"])
    errs["H"] = rel_err(fl.H_natural(cpu(res["H"])), ref["h"])
    errs["V_new"] = rel_err(fl.chunk_rows_to_tokens(VN, chunks, Ttot), ref["V_new"])
    errs["S_T"] = rel_err(cpu(res["S_T"]), ref["S_T"])
    errs["o"] = rel_err(cpu(res["o"]).reshape(ref["o"].shape), ref["o"])
    if res["T"] is not None:
        # k_prep's outputs (inputs of the production pass), natural per chunk:
        # T = A diag(beta), the score block P = (Q K^T) (.) D, the decay rows
        Tn = fl.T_natural(res["T"].detach().cpu().float().numpy())
        Pn = fl.T_natural(res["P"].detach().cpu().float().numpy())
        Rn = res["R"].detach().cpu().double().numpy()
        T_ref, P_ref, R_ref = np.zeros_like(Tn), np.zeros_like(Pn), np.zeros_like(Rn)
        G = ref["G"]
        for c, (_, s0, Lc) in enumerate(chunks):
            A_c = ref["A"][s0:s0 + Lc, :, :Lc].transpose(1, 0, 2)          # [Nv, i, m]
            T_ref[c, :, :Lc, :Lc] = A_c * x["beta"][s0:s0 + Lc].T[:, None, :]
            Gc = G[s0:s0 + Lc].T                                             # [Nv, Lc]
            D = np.tril(np.exp(Gc[:, :, None] - Gc[:, None, :]))
            grp = x["v"].shape[1] // x["q"].shape[1]
            Qc = x["q"][s0:s0 + Lc][:, np.arange(Gc.shape[0]) // grp]        # [Lc, Nv, dk]
            Kc = x["k"][s0:s0 + Lc][:, np.arange(Gc.shape[0]) // grp]
            P_ref[c, :, :Lc, :Lc] = np.einsum("inq,jnq->nij", Qc, Kc) * D
            R_ref[c, :, 0, :Lc] = np.exp(Gc)
            R_ref[c, :, 1, :Lc] = np.exp(Gc[:, -1:] - Gc)
        # fp16 fragments: one rounding of each value (relative 2^-11)
        errs["T"] = rel_err(Tn, T_ref)
        errs["P"] = rel_err(Pn, P_ref)
        errs["R"] = rel_err(Rn, R_ref)
    print(name, {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= tol, (name, key, e)


@pytest.mark.parametrize("name,w,seed,C", KERNEL_CASES[:2], ids=[c[0] for c in KERNEL_CASES[:2]])
def test_fused_path_matches_reference_path(name, w, seed, C):
    """The production call (fp16 matrix-core operands) and the debug call (five
    separate kernels, fp32-level operands) compute the same result; they differ
    by the production path's operand roundings (a few 1e-3 of rms), well inside
    the 2e-2 bound each meets against the oracle."""
    inp = synth.generate(w, seed=seed)
    o1, S1 = run_gpu(inp, out_f32=True)
    res = run_gpu(inp, debug=True, out_f32=True)
    eo = rel_err(o1.cpu().double().numpy(), res["o"].cpu().double().numpy())
    es = rel_err(S1.cpu().double().numpy(), res["S_T"].cpu().double().numpy())
    print(name, "fused vs reference: o %.2e S_T %.2e" % (eo, es), flush=True)
    assert eo < 1e-2 and es < 1e-2
