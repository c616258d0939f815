"""gdr_chunk_fwd_noalloc (per-GPU scratch array, no allocation) against
gdr_chunk_fwd (caller workspace) through the C ABI: the same kernels on the
same inputs give the same bits. Three calls in a row on one GPU, each smaller
than the one before, so that a later call runs on scratch a larger one left
behind."""
import ctypes

import numpy as np
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth

pytestmark = pytest.mark.gpu


def _inputs(cfg):
    w = synth.WORKLOADS[cfg]
    inp = synth.generate(w, seed=cfg)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens")}
    return w, inp, d


def _noalloc(lib, inp, d):
    """gdr_chunk_fwd_noalloc called directly through ctypes."""
    prob, o, S_T, cu_dev, cu_host, scale, ins = api._prepare(
        d["q"], d["k"], d["v"], d["beta"], d["g"], inp["scale"], d["S0"], d["cu_seqlens"], inp["cu_seqlens"], 64,
        True, None, workspace=False)
    q, k, v, beta, g, S0 = ins
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(prob), p(q), p(k), p(v), p(g), p(beta), ctypes.c_float(scale), p(S0),
                                   p(cu_dev), p(cu_host), p(o), p(S_T), ctypes.c_void_p(stream))
    assert st == 0, lib.gdr_last_error_message()
    torch.cuda.synchronize()
    return o, S_T


def test_noalloc_matches_workspace_entry_point_on_successive_calls():
    lib = api.load_library()
    for cfg in (3, 2, 1):                                  # each call smaller than the one before
        w, inp, d = _inputs(cfg)
        p = api.make_problem(inp["q"].shape[0], inp["q"].shape[1], w.Nk, w.Nv, w.dk, w.dv, inp["N"],
                             api.GDR_BF16 if w.dtype == "bf16" else api.GDR_F32)
        assert api.workspace_size(p) <= lib.gdr_chunk_fwd_noalloc_max_workspace()
        o_ref, S_ref = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"],
                                     initial_state=d["S0"], cu_seqlens=d["cu_seqlens"],
                                     cu_seqlens_cpu=inp["cu_seqlens"])
        torch.cuda.synchronize()
        o, S = _noalloc(lib, inp, d)
        rms = float(o_ref.float().pow(2).mean().sqrt())
        diff = float((o.float() - o_ref.float()).abs().max()) / rms
        print("cfg%d (%s): noalloc vs workspace max|d|/rms o %.3e, S_T equal %s" % (
            cfg, w.name, diff, torch.equal(S, S_ref)), flush=True)
        assert torch.equal(o, o_ref), cfg
        assert torch.equal(S, S_ref), cfg
        # the binding's wrapper too
        o2, S2 = api.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"],
                                       initial_state=d["S0"], cu_seqlens=d["cu_seqlens"],
                                       cu_seqlens_cpu=inp["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref) and torch.equal(S2, S_ref), cfg
