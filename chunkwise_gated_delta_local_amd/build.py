"""Build ``_build/libgdr.so`` from ``csrc/`` with hipcc for gfx950.

Every HIP translation unit is compiled with packed fp32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libgdr.so")
SOURCES = ["gdr_api.hip", "gdr_kernels.hip", "gdr_fp16.hip", "gdr_recurrent.hip", "gdr_backward.hip",
           "gdr_peaks.hip"]
# per-file options: the matrix-core loops of these files keep their accumulators
# in VGPRs (without it the compiler moves loop-carried accumulators between
# AGPRs and VGPRs on every iteration)
EXTRA_FLAGS = {"gdr_peaks.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gdr_fp16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(HERE, "csrc", src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msgs = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(msgs)))
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join("%s:\n%s" % f for f in failed))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    try:                                   # every symbol must resolve (a missing kernel stub shows here)
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        os.unlink(tmp)
        raise RuntimeError("built library does not load: %s" % e)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
