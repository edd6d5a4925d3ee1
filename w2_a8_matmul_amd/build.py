"""Build libs3d8.so in-tree: HIP kernels for gfx950 with hipcc, the host
packer with g++, linked by hipcc.  Needs no GPU (hipcc cross-compiles)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libs3d8.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # exact arithmetic: no contraction into FMA, IEEE division, no FTZ
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first kernel arguments arrive in SGPRs at wave start (gfx950
    # kernarg preload) instead of through a scalar load round trip
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-march=x86-64-v3", "-ffp-contract=off",
              "-fno-fast-math", "-pthread", "-I", INCLUDE, "-I", CSRC]


# hipcc hands the target feature above to its host (x86) pass as well, which
# ignores it with this note; the feature is meant for the device pass only and
# the driver offers no device-only form of -Xclang, so the note is dropped
_HOST_PASS_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    err = "".join(line for line in r.stderr.splitlines(keepends=True) if _HOST_PASS_NOTE not in line)
    if err:
        print(err, end="", file=sys.stderr, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def build(verbose: bool = False) -> str:
    """Compile every source and (re)link libs3d8.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        base, ext = os.path.splitext(name)
        obj = os.path.join(BUILD, base + ".o")
        if ext == ".hip":
            _run([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj], verbose)
        elif ext == ".cpp":
            _run(["g++", *HOST_FLAGS, "-c", src, "-o", obj], verbose)
        else:
            continue
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-pthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
