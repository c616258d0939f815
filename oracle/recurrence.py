"""ctypes wrapper around the fp64 token-recurrence oracle (``recurrence.c``).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the bench's
CPU-baseline leg; never by the product path.

The library is compiled with gcc (OpenMP over independent (sequence, V-head)
units). ``build()`` compiles it; ``recurrence()`` compiles it first if no
built library is present.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recurrence.c")
# GDR_ORACLE_LIBRARY names another build (the sanitizer build below)
_LIB = os.environ.get("GDR_ORACLE_LIBRARY") or os.path.join(_HERE, "_build", "liboracle_recurrence.so")
_SAN_LIB = os.path.join(_HERE, "_build_san", "liboracle_recurrence.so")
_libs = {}


def compile_source(src: str, out: str, sanitize: bool = False) -> str:
    """Compile a recurrence source file into a shared library at ``out``; with
    ``sanitize``, single-threaded under AddressSanitizer and
    UndefinedBehaviorSanitizer with the compiler of libgdr.so's sanitizer
    build (one sanitizer runtime serves both in a process)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined",
               "-fno-omit-frame-pointer", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = True, sanitize: bool = False) -> str:
    out = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out):
        compile_source(_SRC, out, sanitize)
    return out


def _load(path: Optional[str] = None):
    path = path or _LIB
    if path not in _libs:
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        f = lib.gdr_oracle_recurrence
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double, P, ctypes.c_int32, P, P, P,
                      ctypes.c_int32, P]
        f.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def recurrence(q, k, v, beta, g=None, scale=None, S0=None, cu_seqlens=None,
               literal_undecayed_read=False, unit_mask=None, threads: Optional[int] = None,
               lib_path: Optional[str] = None):
    """Run the token recurrence in fp64.

    q, k: [Ttot, Nk, dk]; v: [Ttot, Nv, dv]; beta, g: [Ttot, Nv]; S0: [N, Nv, dk, dv].
    A leading batch axis [B, T, ...] is accepted when cu_seqlens is None (each
    batch row is one sequence). Returns (o [.., Nv, dv], S_T [N, Nv, dk, dv]) in fp64.
    unit_mask: optional bool array [N, Nv]; skipped units are returned as NaN.
    threads: OpenMP team size (default: the runtime's). lib_path: load another
    build of the same source (the mutation tests use planted-mistake copies).
    """
    q, k, v, beta, g, S0 = (_f64(x) for x in (q, k, v, beta, g, S0))
    lead = q.shape[:-2]
    if cu_seqlens is None:
        if q.ndim == 4:
            B, T = q.shape[0], q.shape[1]
        else:
            B, T = 1, q.shape[0]
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
    Nk, dk = q.shape[-2], q.shape[-1]
    Nv, dv = v.shape[-2], v.shape[-1]
    Ttot = int(np.prod(lead))
    N = len(cu) - 1
    q2, k2 = q.reshape(Ttot, Nk, dk), k.reshape(Ttot, Nk, dk)
    v2 = v.reshape(Ttot, Nv, dv)
    b2 = beta.reshape(Ttot, Nv)
    g2 = None if g is None else g.reshape(Ttot, Nv)
    if S0 is not None:
        S0 = S0.reshape(N, Nv, dk, dv)
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(N, Nv))
    o = np.full((Ttot, Nv, dv), np.nan)
    ST = np.full((N, Nv, dk, dv), np.nan)
    if scale is None:
        scale = dk ** -0.5
    lib = _load(lib_path)
    used = ctypes.c_int32(0)
    rc = lib.gdr_oracle_recurrence(Ttot, Nk, Nv, dk, dv, N, _ptr(cu), _ptr(q2), _ptr(k2), _ptr(v2),
                                   _ptr(g2), _ptr(b2), float(scale), _ptr(S0),
                                   1 if literal_undecayed_read else 0, _ptr(mask), _ptr(o), _ptr(ST),
                                   int(threads or 0), ctypes.byref(used))
    recurrence.last_threads = int(used.value)
    if rc != 0:
        raise ValueError("oracle recurrence rejected its arguments")
    return o.reshape(*lead, Nv, dv), ST
