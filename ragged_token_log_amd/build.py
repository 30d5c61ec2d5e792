"""Builds liblogprob.so in-tree for gfx950.

    python -m ragged_token_log_amd.build

The host plan (plain C++) is compiled with g++, the device code with hipcc
for gfx950, and both are linked into ``ragged_token_log_amd/liblogprob.so``.
Packed fp32 instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblogprob.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    plan_o = os.path.join(BUILD, "plan.o")
    kern_o = os.path.join(BUILD, "logprob_kernels.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc, "-c",
          os.path.join(CSRC, "plan.cpp"), "-o", plan_o], verbose)
    hipcc = _hipcc()
    _run([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "logprob_kernels.hip"),
          "-o", kern_o], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", plan_o, kern_o, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
