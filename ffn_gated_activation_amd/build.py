"""Compile libsitu_glu.so in-tree for gfx950.

    python -m ffn_gated_activation_amd.build

The host API (csrc/situ_glu_api.cpp, plain C++) is compiled with g++, the
kernels (csrc/situ_glu_kernels.hip) with hipcc for gfx950, and both are linked
into ffn_gated_activation_amd/libsitu_glu.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsitu_glu.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # fp32 denormals are kept (no flush to zero)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsitu_glu.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_library(verbose: bool = False, extra_hipcc: list[str] | None = None, out: str = LIB,
                  build_dir: str = BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    api_o = os.path.join(build_dir, "situ_glu_api.o")
    ker_o = os.path.join(build_dir, "situ_glu_kernels.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
          os.path.join(CSRC, "situ_glu_api.cpp"), "-o", api_o], verbose)
    _run([_hipcc(), *HIPCC_FLAGS, *(extra_hipcc or []), "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "situ_glu_kernels.hip"), "-o", ker_o], verbose)
    tmp = out + ".tmp%d" % os.getpid()
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, api_o, ker_o], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-q" not in sys.argv))
