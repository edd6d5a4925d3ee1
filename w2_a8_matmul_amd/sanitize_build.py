"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, for
the CPU tests (tests/test_sanitized_host.py).

Builds, under _build/sanitize/:
  libs3d8_san.so     the library with its host code (the packer, the ABI's
                     argument validation and launch glue) instrumented; the
                     device code is built as usual (GPU sanitizers are not
                     used), so only host memory errors and undefined
                     behaviour are caught;
  liboracle_san.so   the oracle, instrumented.
Everything is compiled by the ROCm clang, so one sanitizer runtime (clang's
shared ASan runtime, which also carries UBSan) serves both; a Python process
loads it with LD_PRELOAD and selects the two libraries with S3D8_LIB and
ORACLE_LIB (see sanitizer_env).  Needs no GPU.
"""
from __future__ import annotations

import glob
import os

from . import build as _b

SAN_DIR = os.path.join(_b.BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libs3d8_san.so")
SAN_ORACLE = os.path.join(SAN_DIR, "liboracle_san.so")
LLVM = "/opt/rocm/llvm"
CLANGXX = os.path.join(LLVM, "bin", "clang++")
CLANG = os.path.join(LLVM, "bin", "clang")
ORACLE_SRC = os.path.join(_b.ROOT, "oracle", "oracle.c")

# host-side instrumentation only: on the device compiler's command line each
# sanitizer flag is scoped to the host pass
_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    libs = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not libs:
        raise FileNotFoundError("clang's shared ASan runtime is not installed under " + LLVM)
    return libs[-1]


def _stale(out, srcs):
    return not os.path.exists(out) or any(os.path.getmtime(s) > os.path.getmtime(out) for s in srcs)


def build_sanitized(verbose: bool = False):
    """Build both sanitized libraries (skipped when newer than their sources);
    returns (library, oracle library)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    hip = os.path.join(_b.CSRC, "s3d8_kernels.hip")
    cpp = os.path.join(_b.CSRC, "s3d8_host.cpp")
    hdrs = glob.glob(os.path.join(_b.CSRC, "*.h")) + glob.glob(os.path.join(_b.INCLUDE, "*.h"))
    if _stale(SAN_LIB, [hip, cpp, *hdrs]):
        k_o, h_o = os.path.join(SAN_DIR, "k.o"), os.path.join(SAN_DIR, "h.o")
        dev_flags = [f for f in _b.HIP_FLAGS if f != "-O3"]
        _b._run([_b.HIPCC, *dev_flags, "-O1", "-g", *_HOST_SAN, "-c", hip, "-o", k_o], verbose)
        _b._run([CLANGXX, "-O1", "-g", "-fPIC", "-std=c++17", "-ffp-contract=off", "-pthread", *_SAN,
                 "-I", _b.INCLUDE, "-I", _b.CSRC, "-c", cpp, "-o", h_o], verbose)
        tmp = SAN_LIB + ".tmp%d" % os.getpid()
        _b._run([CLANGXX, "-shared", "-fPIC", *_SAN, "-shared-libasan", "-o", tmp, k_o, h_o,
                 "-L/opt/rocm/lib", "-lamdhip64", "-pthread", "-Wl,-rpath,/opt/rocm/lib"], verbose)
        os.replace(tmp, SAN_LIB)
    if _stale(SAN_ORACLE, [ORACLE_SRC]):
        tmp = SAN_ORACLE + ".tmp%d" % os.getpid()
        _b._run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", *_SAN,
                 "-shared-libasan", "-o", tmp, ORACLE_SRC, "-lm", "-Wl,-rpath," + os.path.join(LLVM, "lib")],
                verbose)
        os.replace(tmp, SAN_ORACLE)
    return SAN_LIB, SAN_ORACLE


def sanitizer_env(base=None) -> dict:
    """Environment for a Python process that runs the library and the oracle
    under the sanitizers (halting on the first report)."""
    env = dict(os.environ if base is None else base)
    env.update({
        "S3D8_LIB": SAN_LIB,
        "ORACLE_LIB": SAN_ORACLE,
        "LD_PRELOAD": asan_runtime(),
        "LD_LIBRARY_PATH": os.path.join(LLVM, "lib") + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH")
                                                        else ""),
        # Python itself is not instrumented and keeps memory to exit: no leak report
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    return env


if __name__ == "__main__":
    print(build_sanitized(verbose=True))
