"""Host-side sanitizer run, CPU only (no GPU is touched).

Builds libgdr.so with its host code under AddressSanitizer and
UndefinedBehaviorSanitizer (the device code as in the normal build) and the
oracle's C token recurrence under both, then runs the C-ABI tests and the
oracle's pins against those builds in a child process with the sanitizer
runtime preloaded. Any sanitizer report fails the run.

    python tests/sanitize_cpu.py            # build both, then test
    python tests/sanitize_cpu.py --no-build # test the existing builds
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["tests/test_abi_cpu.py", "tests/test_oracle_pins.py"]


def main() -> int:
    sys.path.insert(0, ROOT)
    import importlib
    from chunkwise_gated_delta_local_amd import build as gbuild
    recurrence = importlib.import_module("oracle.recurrence")
    lib = os.path.join(gbuild.SAN_BUILD_DIR, "libgdr.so")
    olib = recurrence._SAN_LIB
    if "--no-build" not in sys.argv:
        print("building", gbuild.build(sanitize=True), flush=True)
        print("building", recurrence.build(force=True, sanitize=True), flush=True)
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        print("no AddressSanitizer runtime found")
        return 2
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtimes[-1],
        # the interpreter is not instrumented: its own allocations are not tracked for leaks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "GDR_LIBRARY": lib,
        "GDR_ORACLE_LIBRARY": olib,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    print(" ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
