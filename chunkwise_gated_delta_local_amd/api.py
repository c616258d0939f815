"""Thin ctypes binding of ``libgdr.so`` (include/gdr.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels. If
the library has not been built, every call raises immediately: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# GDR_LIBRARY names another build of the same library (the host-sanitizer
# build that tests/sanitize_cpu.py makes); the default is the in-tree build
_LIB_PATH = os.environ.get("GDR_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build",
                                                          "libgdr.so")
_lib = None

GDR_F32, GDR_BF16 = 0, 1
NUM_STAGES = 6
STAGE_NAMES = ("chunk_table", "gate_cumsum", "build_solve", "wu", "state", "output")
BWD_NUM_STAGES = 5
BWD_STAGE_NAMES = ("forward_recompute", "k_bwd_prep", "k_bwd_state", "k_bwd_chunk", "k_bwd_reduce_qk")
_DTYPES = {torch.float32: GDR_F32, torch.bfloat16: GDR_BF16}

EXPORTED = ("gdr_validate", "gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd_debug_workspace_size",
            "gdr_chunk_fwd", "gdr_chunk_fwd_debug", "gdr_chunk_fwd_timed", "gdr_recurrent_fwd",
            "gdr_chunk_fwd_segmented_workspace_size", "gdr_chunk_fwd_segmented",
            "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd",
            "gdr_status_string", "gdr_last_error_message",
            "gdr_peak_copy", "gdr_peak_mfma", "gdr_peak_mfma_flops",
            "gdr_chunk_fwd_noalloc", "gdr_chunk_fwd_noalloc_max_workspace")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class Intermediates(ctypes.Structure):
    _fields_ = [("G", ctypes.c_void_p), ("A", ctypes.c_void_p), ("W", ctypes.c_void_p),
                ("U", ctypes.c_void_p), ("KT", ctypes.c_void_p), ("H", ctypes.c_void_p),
                ("VN", ctypes.c_void_p), ("T", ctypes.c_void_p), ("P", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("num_chunks", ctypes.c_int64)]


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("gdr status %d: %s" % (status, message))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdr.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libgdr.so is not built (%s); run __graft_entry__.build() first" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, PP = ctypes.c_void_p, ctypes.POINTER(Problem)
    fwd_args = [PP, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdr_validate.argtypes = [PP, P]
    lib.gdr_chunk_fwd_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd_debug_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd.argtypes = fwd_args
    lib.gdr_chunk_fwd_debug.argtypes = fwd_args + [ctypes.POINTER(Intermediates)]
    lib.gdr_chunk_fwd_timed.argtypes = fwd_args + [P]
    lib.gdr_recurrent_fwd.argtypes = [PP, P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_int, P, P, P]
    lib.gdr_chunk_fwd_segmented_workspace_size.argtypes = [PP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd_segmented.argtypes = fwd_args[:12] + [ctypes.c_int32] + fwd_args[12:] + [P]
    lib.gdr_chunk_bwd_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_bwd.argtypes = fwd_args[:10] + [P] * 8 + [P, ctypes.c_size_t, P, P]
    for f in ("gdr_validate", "gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd_debug_workspace_size",
              "gdr_chunk_fwd", "gdr_chunk_fwd_debug", "gdr_chunk_fwd_timed", "gdr_recurrent_fwd",
              "gdr_chunk_fwd_segmented_workspace_size", "gdr_chunk_fwd_segmented",
              "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd"):
        getattr(lib, f).restype = ctypes.c_int
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error_message.argtypes = []
    lib.gdr_last_error_message.restype = ctypes.c_char_p
    lib.gdr_chunk_fwd_noalloc.argtypes = fwd_args[:12] + [P]
    lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_fwd_noalloc_max_workspace.argtypes = []
    lib.gdr_chunk_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.gdr_peak_copy.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int32, P]
    lib.gdr_peak_copy.restype = ctypes.c_int
    lib.gdr_peak_mfma.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P]
    lib.gdr_peak_mfma.restype = ctypes.c_int
    lib.gdr_peak_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.gdr_peak_mfma_flops.restype = ctypes.c_double
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise GdrError(status, lib.gdr_last_error_message().decode())


def make_problem(batch, seq_len, Nk, Nv, dk, dv, num_seqs, io_dtype=GDR_BF16, beta_dtype=None,
                 chunk_size=64, out_dtype=None) -> Problem:
    return Problem(int(batch), int(seq_len), int(Nk), int(Nv), int(dk), int(dv), int(chunk_size),
                   int(num_seqs), int(io_dtype), int(io_dtype if beta_dtype is None else beta_dtype),
                   int(io_dtype if out_dtype is None else out_dtype))


def validate(problem: Problem, cu_seqlens_host=None) -> int:
    """Host-only validation; returns the status code (0 = ok)."""
    lib = load_library()
    cu = None
    if cu_seqlens_host is not None:
        cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    return lib.gdr_validate(ctypes.byref(problem), None if cu is None else ctypes.c_void_p(cu.data_ptr()))


def workspace_size(problem: Problem, debug: bool = False, segment_chunks: Optional[int] = None) -> int:
    """Workspace bytes of gdr_chunk_fwd, of gdr_chunk_fwd_debug (debug), or of
    gdr_chunk_fwd_segmented with that segment_chunks (0: automatic)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    if segment_chunks is not None:
        _check(lib.gdr_chunk_fwd_segmented_workspace_size(ctypes.byref(problem), ctypes.c_int32(segment_chunks),
                                                          ctypes.byref(n)))
        return int(n.value)
    fn = lib.gdr_chunk_fwd_debug_workspace_size if debug else lib.gdr_chunk_fwd_workspace_size
    _check(fn(ctypes.byref(problem), ctypes.byref(n)))
    return int(n.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _aligned16(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """The library takes tensors whose base address is 16-byte aligned; a
    contiguous view that starts elsewhere (a one-token slice of a decode
    batch, say) is passed as an aligned copy."""
    if t is None or t.data_ptr() % 16 == 0:
        return t
    return t.clone(memory_format=torch.contiguous_format)


_GUARD_BYTE = 0xA5


def _guarded(nbytes, guard, dev):
    """A uint8 buffer of nbytes with `guard` canary bytes (0xA5) before and
    after it: returns (whole buffer, the inner part)."""
    whole = torch.empty(nbytes + 2 * guard, dtype=torch.uint8, device=dev)
    whole[:guard].fill_(_GUARD_BYTE)
    whole[guard + nbytes:].fill_(_GUARD_BYTE)
    return whole, whole[guard:guard + nbytes]


def _check_guards(guards, guard):
    """Raise if a kernel wrote into the canary bytes around a buffer."""
    for name, whole in guards:
        n = whole.numel() - 2 * guard
        for part, band in (("before", whole[:guard]), ("after", whole[guard + n:])):
            bad = (band != _GUARD_BYTE).nonzero()
            if bad.numel():
                raise RuntimeError("write %s the %s buffer: %d canary bytes changed, first at offset %d"
                                   % (part, name, bad.numel(), int(bad[0])))


def _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens, cu_seqlens_cpu, chunk_size,
             output_final_state, out_dtype, debug=False, workspace=True, segment_chunks=None, guard=0):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [B,T,Nk,dk] and v [B,T,Nv,dv]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bfloat16 or float32")
    B, T, Nk, dk = q.shape
    Nv, dv = v.shape[2], v.shape[3]
    if beta.shape != (B, T, Nv) or beta.dtype not in (q.dtype, torch.float32):
        raise ValueError("beta must be [B,T,Nv] in the io dtype or float32")
    if g is not None and (g.shape != (B, T, Nv) or g.dtype != torch.float32):
        raise ValueError("g must be [B,T,Nv] float32")
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        cu_host = (cu_seqlens_cpu if cu_seqlens_cpu is not None else cu_seqlens).detach().to(
            "cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens.detach().to(dev, torch.int32).contiguous()
        N = cu_host.numel() - 1
    else:
        N = B
    if initial_state is not None and (initial_state.shape != (N, Nv, dk, dv) or initial_state.dtype != torch.float32):
        raise ValueError("initial_state must be [N,Nv,dk,dv] float32")
    tensors = [q, k, v, beta, g, initial_state]
    for t in tensors:
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous and on the same device")
    q, k, v, beta, g, initial_state = (_aligned16(t) for t in tensors)
    if scale is None:
        scale = dk ** -0.5
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in (q.dtype, torch.float32):
        raise ValueError("out_dtype must be the io dtype or float32")
    prob = make_problem(B, T, Nk, Nv, dk, dv, N, _DTYPES[q.dtype], _DTYPES[beta.dtype], chunk_size,
                        _DTYPES[out_dtype])
    guards = []
    if guard:                                 # debug canaries around every buffer the call writes
        if guard % 256:
            raise ValueError("guard must be a multiple of 256 bytes")
        ob = torch.empty((), dtype=out_dtype).element_size() * v.numel()
        whole, inner = _guarded(ob, guard, dev)
        o = inner.view(out_dtype).view(v.shape)
        guards.append(("o", whole))
        S_T = None
        if output_final_state:
            whole, inner = _guarded(4 * N * Nv * dk * dv, guard, dev)
            S_T = inner.view(torch.float32).view((N, Nv, dk, dv))
            guards.append(("final state", whole))
    else:
        o = torch.empty(v.shape, dtype=out_dtype, device=dev)
        S_T = torch.empty((N, Nv, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    if not workspace:                         # token-by-token path: no workspace
        return prob, o, S_T, cu_dev, cu_host, scale, (q, k, v, beta, g, initial_state)
    if guard:
        whole, ws = _guarded(workspace_size(prob, debug, segment_chunks), guard, dev)
        guards.append(("workspace", whole))
    else:
        ws = torch.empty(workspace_size(prob, debug, segment_chunks), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.c_float(scale),
            _ptr(initial_state), _ptr(cu_dev), _ptr(cu_host), _ptr(o), _ptr(S_T), _ptr(ws),
            ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream)]
    if segment_chunks is not None:            # gdr_chunk_fwd_segmented: segment_chunks before the workspace
        args = args[:12] + [ctypes.c_int32(segment_chunks)] + args[12:]
    keep = (cu_dev, cu_host, ws, q, k, v, beta, g, initial_state, guards)
    return prob, args, o, S_T, keep


def chunk_fwd(q, k, v, beta, g=None, scale=None, initial_state=None, output_final_state=True,
              cu_seqlens=None, cu_seqlens_cpu=None, chunk_size=64, out_dtype=None, segment_chunks=None,
              guard=0):
    """Chunked gated delta-rule forward. Returns (o, final_state or None).

    out_dtype: dtype of o, the io dtype (default) or torch.float32.
    segment_chunks: None runs gdr_chunk_fwd (one serial state pass per
    sequence); an int runs gdr_chunk_fwd_segmented with segments of that many
    chunks (0: the library chooses).
    guard: debugging aid, off by default. With guard > 0 (a multiple of 256)
    the workspace, o and the final state are placed between `guard` canary
    bytes on either side; after the call (which then synchronises) a changed
    canary byte raises RuntimeError naming the buffer."""
    lib = load_library()
    prob, args, o, S_T, keep = _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens, cu_seqlens_cpu,
                                        chunk_size, output_final_state, out_dtype, segment_chunks=segment_chunks,
                                        guard=guard)
    if segment_chunks is None:
        _check(lib.gdr_chunk_fwd(*args))
    else:
        _check(lib.gdr_chunk_fwd_segmented(*args, None))
    if guard:
        torch.cuda.synchronize(q.device)
        _check_guards(keep[-1], guard)
    del keep
    return o, S_T


def chunk_fwd_noalloc(q, k, v, beta, g=None, scale=None, initial_state=None, output_final_state=True,
                      cu_seqlens=None, cu_seqlens_cpu=None, chunk_size=64, out_dtype=None):
    """As chunk_fwd, through gdr_chunk_fwd_noalloc: the library's per-GPU
    scratch array serves as the workspace (o and the final state are still
    allocated here, by torch). Calls on one GPU must not overlap."""
    lib = load_library()
    prob, o, S_T, cu_dev, cu_host, scale, ins = _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens,
                                                         cu_seqlens_cpu, chunk_size, output_final_state,
                                                         out_dtype, workspace=False)
    q, k, v, beta, g, initial_state = ins
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib.gdr_chunk_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     ctypes.c_float(scale), _ptr(initial_state), _ptr(cu_dev), _ptr(cu_host),
                                     _ptr(o), _ptr(S_T), ctypes.c_void_p(stream)))
    return o, S_T


def recurrent_fwd(q, k, v, beta, g=None, scale=None, initial_state=None, output_final_state=True,
                  cu_seqlens=None, cu_seqlens_cpu=None, use_qk_l2norm_in_kernel=False, out_dtype=None):
    """Token-by-token (fused recurrent) gated delta-rule forward: the same
    result as chunk_fwd, for decoding and short inputs. Returns (o, final_state
    or None). use_qk_l2norm_in_kernel: q and k are L2-normalised per token
    inside the kernel."""
    lib = load_library()
    prob, o, S_T, cu_dev, cu_host, scale, ins = _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens,
                                                         cu_seqlens_cpu, 64, output_final_state, out_dtype,
                                                         workspace=False)
    q, k, v, beta, g, initial_state = ins
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib.gdr_recurrent_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 ctypes.c_float(scale), _ptr(initial_state), _ptr(cu_dev), _ptr(cu_host),
                                 ctypes.c_int(1 if use_qk_l2norm_in_kernel else 0), _ptr(o), _ptr(S_T),
                                 ctypes.c_void_p(stream)))
    del cu_dev, cu_host
    return o, S_T


class Backward:
    """A prepared gdr_chunk_bwd call on fixed tensors, for repeated launches.
    Gradient buffers (fp32) and the workspace are allocated once; each call
    enqueues the whole backward (forward recompute included) on the stream
    that was current at construction. d_o has o's dtype: the io dtype, or
    float32 (out_dtype)."""

    def __init__(self, q, k, v, beta, g=None, scale=None, initial_state=None, cu_seqlens=None,
                 cu_seqlens_cpu=None, d_o=None, d_final_state=None, chunk_size=64, want_dg=True,
                 want_dh0=True):
        self.lib = load_library()
        if d_o is None or d_o.shape != v.shape or d_o.dtype not in (q.dtype, torch.float32):
            raise ValueError("d_o must be shaped like v, in the io dtype or float32")
        prob, _o, _S, cu_dev, cu_host, scale, ins = _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens,
                                                             cu_seqlens_cpu, chunk_size, False, d_o.dtype,
                                                             workspace=False)
        q, k, v, beta, g, initial_state = ins
        N = prob.num_seqs
        B, T, Nk, dk = q.shape
        Nv, dv = v.shape[2], v.shape[3]
        if d_final_state is not None and (d_final_state.shape != (N, Nv, dk, dv)
                                          or d_final_state.dtype != torch.float32):
            raise ValueError("d_final_state must be [N,Nv,dk,dv] float32")
        for t in (d_o, d_final_state):
            if t is not None and (t.device != q.device or not t.is_contiguous()):
                raise ValueError("all tensors must be contiguous and on the same device")
        d_o, d_final_state = _aligned16(d_o), _aligned16(d_final_state)
        dev = q.device
        f32 = dict(dtype=torch.float32, device=dev)
        self.dq = torch.empty(q.shape, **f32)
        self.dk = torch.empty(k.shape, **f32)
        self.dv = torch.empty(v.shape, **f32)
        self.dbeta = torch.empty(beta.shape, **f32)
        self.dg = torch.empty(beta.shape, **f32) if want_dg else None
        self.dh0 = torch.empty((N, Nv, dk, dv), **f32) if want_dh0 else None
        n = ctypes.c_size_t(0)
        self.problem = prob
        _check(self.lib.gdr_chunk_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
        self.ws = torch.empty(int(n.value), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        self.args = [ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.c_float(scale),
                     _ptr(initial_state), _ptr(cu_dev), _ptr(cu_host), _ptr(d_o), _ptr(d_final_state),
                     _ptr(self.dq), _ptr(self.dk), _ptr(self.dv), _ptr(self.dbeta), _ptr(self.dg),
                     _ptr(self.dh0), _ptr(self.ws), ctypes.c_size_t(self.ws.numel()), ctypes.c_void_p(stream)]
        self._keep = (q, k, v, beta, g, initial_state, d_o, d_final_state, cu_dev, cu_host)

    def __call__(self):
        _check(self.lib.gdr_chunk_bwd(*self.args, None))

    def timed(self, events):
        """Enqueue one backward and record the BWD_NUM_STAGES + 1
        torch.cuda.Event objects around its stages (recorded once beforehand,
        so that their HIP handles exist); a None entry is not recorded."""
        if len(events) != BWD_NUM_STAGES + 1:
            raise ValueError("timed() takes %d events, got %d" % (BWD_NUM_STAGES + 1, len(events)))
        handles = (ctypes.c_void_p * (BWD_NUM_STAGES + 1))(*[None if e is None else e.cuda_event for e in events])
        _check(self.lib.gdr_chunk_bwd(*self.args, handles))


def chunk_bwd(q, k, v, beta, d_o, g=None, scale=None, initial_state=None, d_final_state=None,
              cu_seqlens=None, cu_seqlens_cpu=None, chunk_size=64):
    """Backward of chunk_fwd: returns dict dq, dk, dv, dbeta, dg, dh0 (fp32),
    the gradients of a loss given dL/do (d_o) and dL/dS_T (d_final_state,
    None = zeros). The forward is recomputed. With g None, dg is the
    gradient at g = 0."""
    bwd = Backward(q, k, v, beta, g=g, scale=scale, initial_state=initial_state, cu_seqlens=cu_seqlens,
                   cu_seqlens_cpu=cu_seqlens_cpu, d_o=d_o, d_final_state=d_final_state, chunk_size=chunk_size)
    bwd()
    return dict(dq=bwd.dq, dk=bwd.dk, dv=bwd.dv, dbeta=bwd.dbeta, dg=bwd.dg, dh0=bwd.dh0)


def num_chunks(B, T, cu_host, chunk_size=64) -> int:
    C = int(chunk_size)
    if cu_host is None:
        return B * ((T + C - 1) // C)
    lens = (cu_host[1:] - cu_host[:-1]).tolist()
    return sum((n + C - 1) // C for n in lens)


def chunk_fwd_debug(q, k, v, beta, g=None, scale=None, initial_state=None, output_final_state=True,
                    cu_seqlens=None, cu_seqlens_cpu=None, chunk_size=64, out_dtype=None):
    """As chunk_fwd, plus the kernels' intermediates in their stored layouts
    (include/gdr.h, gdr_intermediates_t). Returns a dict."""
    lib = load_library()
    prob, args, o, S_T, keep = _prepare(q, k, v, beta, g, scale, initial_state, cu_seqlens, cu_seqlens_cpu,
                                        chunk_size, output_final_state, out_dtype, debug=True)
    B, T, Nk, dk = q.shape
    Nv, dv = v.shape[2], v.shape[3]
    C = int(chunk_size)
    NT = num_chunks(B, T, keep[1], C)
    ntb, ntp = C // 16, max(1, C // 32)
    dev, dt = q.device, q.dtype
    out = dict(
        G=torch.zeros((B * T, Nv), dtype=torch.float32, device=dev),
        A=torch.zeros((B * T, Nv, C), dtype=torch.float32, device=dev),
        W=torch.zeros((NT, Nv, ntb, dk // 32, 64, 8), dtype=torch.float32, device=dev),
        U=torch.zeros((NT, Nv, ntb, dv // 16, 64, 4), dtype=torch.float32, device=dev),
        KT=torch.zeros((NT, Nk, dk // 16, ntp, 64, 8), dtype=dt, device=dev),
        H=torch.zeros((NT, Nv, dv // 16, dk // 32, 64, 8), dtype=torch.float32, device=dev),
        VN=torch.zeros((NT, Nv, dv // 16, ntp, 64, 8), dtype=torch.float32, device=dev),
    )
    fp16_path = dt == torch.bfloat16 and C == 64
    out.update(
        T=torch.zeros((NT, Nv, 6, 64, 8), dtype=torch.float16, device=dev) if fp16_path else None,
        P=torch.zeros((NT, Nv, 6, 64, 8), dtype=torch.float16, device=dev) if fp16_path else None,
        R=torch.zeros((NT, Nv, 2, 64), dtype=torch.float32, device=dev) if fp16_path else None,
    )
    dbg = Intermediates(*(_ptr(out[n]) for n in ("G", "A", "W", "U", "KT", "H", "VN", "T", "P", "R")), 0)
    _check(lib.gdr_chunk_fwd_debug(*args, ctypes.byref(dbg)))
    out.update(o=o, S_T=S_T, num_chunks=int(dbg.num_chunks))
    del keep
    return out


class Forward:
    """A prepared gdr_chunk_fwd call on fixed tensors, for repeated launches
    (benchmarks). Outputs and workspace are allocated once; each call enqueues
    the whole forward on the stream that was current at construction."""

    def __init__(self, q, k, v, beta, g=None, scale=None, initial_state=None, output_final_state=True,
                 cu_seqlens=None, cu_seqlens_cpu=None, chunk_size=64, out_dtype=None, segment_chunks=None,
                 five_kernel=False):
        """five_kernel: run the five kernels as separate launches (through
        gdr_chunk_fwd_debug with no intermediates requested) even where
        gdr_chunk_fwd would take the fused path; such calls record no stage
        events."""
        self.lib = load_library()
        self.segment_chunks = segment_chunks
        self.five_kernel = five_kernel
        if five_kernel and segment_chunks is not None:
            raise ValueError("five_kernel and segment_chunks do not combine")
        self.problem, self.args, self.o, self.final_state, self._keep = _prepare(
            q, k, v, beta, g, scale, initial_state, cu_seqlens, cu_seqlens_cpu, chunk_size,
            output_final_state, out_dtype, debug=five_kernel, segment_chunks=segment_chunks)
        self._no_intermediates = Intermediates()
        self.stage_events = not five_kernel
        self.inputs = (q, k, v, beta, g, initial_state)       # keep alive while prepared

    def __call__(self):
        if self.five_kernel:
            _check(self.lib.gdr_chunk_fwd_debug(*self.args, ctypes.byref(self._no_intermediates)))
        elif self.segment_chunks is None:
            _check(self.lib.gdr_chunk_fwd(*self.args))
        else:
            _check(self.lib.gdr_chunk_fwd_segmented(*self.args, None))

    def timed(self, events):
        """Enqueue one forward and record the NUM_STAGES + 1 torch.cuda.Event
        objects around its stages (they must have been recorded once, so that
        their HIP handles exist); a None entry is not recorded."""
        if len(events) != NUM_STAGES + 1:
            raise ValueError("timed() takes %d events, got %d" % (NUM_STAGES + 1, len(events)))
        handles = (ctypes.c_void_p * (NUM_STAGES + 1))(*[None if e is None else e.cuda_event for e in events])
        if self.segment_chunks is None:
            _check(self.lib.gdr_chunk_fwd_timed(*self.args, handles))
        else:
            _check(self.lib.gdr_chunk_fwd_segmented(*self.args, handles))
