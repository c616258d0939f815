"""Shared helpers of the GPU tests: run the HIP path, run the oracle, compare."""
import numpy as np
import torch

from chunkwise_gated_delta_local_amd import api

TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_err(x, ref):
    """max |x - ref| / rms(ref)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(x - ref)) / (rms if rms > 0 else 1.0))


def to_dev(inp, beta_f32=False):
    d = {}
    for key in ("q", "k", "v", "beta", "g", "S0", "cu_seqlens"):
        t = inp[key]
        if t is not None:
            if key == "beta" and beta_f32:
                t = t.float()
            t = t.cuda()
        d[key] = t
    return d


def run_gpu(inp, debug=False, beta_f32=False, output_final_state=True, out_f32=False, chunk_size=64):
    d = to_dev(inp, beta_f32)
    fn = api.chunk_fwd_debug if debug else api.chunk_fwd
    res = fn(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
             output_final_state=output_final_state, cu_seqlens=d["cu_seqlens"],
             cu_seqlens_cpu=inp["cu_seqlens"], out_dtype=torch.float32 if out_f32 else None,
             chunk_size=chunk_size)
    torch.cuda.synchronize()
    return res


def f64(t):
    return None if t is None else t.detach().cpu().double().numpy()


def oracle_inputs(inp):
    """The exact values the GPU sees (io-dtype rounded), in fp64, token-flattened."""
    q, k, v, beta = (f64(inp[n]) for n in ("q", "k", "v", "beta"))
    B, T = q.shape[:2]
    cu = inp["cu_seqlens"]
    cu = np.arange(B + 1) * T if cu is None else cu.numpy()
    g = f64(inp["g"])
    flat = lambda x: None if x is None else x.reshape((B * T,) + x.shape[2:])
    return dict(q=flat(q), k=flat(k), v=flat(v), beta=flat(beta), g=flat(g), S0=f64(inp["S0"]), cu=cu,
                scale=inp["scale"])


def bf16_round(x):
    """Round fp64 values to the nearest bf16 (ties to even), through fp32."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = x32.view(np.uint32).astype(np.uint64)
    r = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def bf16_rounding_excess(o_bf16, o_ref):
    """max over elements of (|o - ref| - |rne_bf16(ref) - ref|) / rms(ref): how
    far the bf16 output lies beyond the error of the correctly rounded exact
    value. A bf16 output is rne(y) of an internal fp32 value y, and
    |rne(y) - ref| <= |rne(ref) - ref| + 2 |y - ref|, so this is at most twice
    the fp32-output error; the tests hold it to the same bound."""
    o = np.asarray(o_bf16, dtype=np.float64)
    ref = np.asarray(o_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(o - ref) - np.abs(bf16_round(ref) - ref)) / (rms if rms > 0 else 1.0))
