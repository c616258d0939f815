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


# host-sanitizer build (tests/sanitize_cpu.py): the host code under AddressSanitizer
# and UndefinedBehaviorSanitizer, the device code as in the normal build
SAN_BUILD_DIR = os.path.join(HERE, "_build_san")
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out_dir = SAN_BUILD_DIR if sanitize else BUILD_DIR
    lib_path = os.path.join(out_dir, "libgdr.so")
    os.makedirs(out_dir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), *(SAN_FLAGS if sanitize else []),
               "-c", os.path.join(HERE, "csrc", src), "-o", obj]
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
    tmp = lib_path + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        link[4:4] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.check_call(link)
    if not sanitize:                       # (the sanitizer build needs its runtime preloaded to load)
        try:                               # every symbol must resolve (a missing kernel stub shows here)
            ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        except OSError as e:
            os.unlink(tmp)
            raise RuntimeError("built library does not load: %s" % e)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
