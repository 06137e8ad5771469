"""Compile libsitu_glu.so in-tree for gfx950.

    python -m ffn_gated_activation_amd.build

The host API (csrc/situ_glu_api.cpp, plain C++) is compiled with g++, the
kernels (csrc/situ_glu_kernels.hip: forward and backward; csrc/situ_glu_mx.hip:
MXFP8 forward and block quantiser; csrc/situ_glu_attn_res.hip:
attention-residual mixing; csrc/situ_glu_gemm.hip: fused grouped FC1 GEMM +
SiTU-GLU on the matrix cores) with hipcc for gfx950, in parallel, and all are
linked into ffn_gated_activation_amd/libsitu_glu.so.
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


HIP_SOURCES = ("situ_glu_kernels.hip", "situ_glu_mx.hip", "situ_glu_attn_res.hip", "situ_glu_gemm.hip")


def build_library(verbose: bool = False, extra_hipcc: list[str] | None = None, out: str = LIB,
                  build_dir: str = BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    api_o = os.path.join(build_dir, "situ_glu_api.o")
    cmds = [["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
             os.path.join(CSRC, "situ_glu_api.cpp"), "-o", api_o]]
    objs = [api_o]
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmds.append([_hipcc(), *HIPCC_FLAGS, *(extra_hipcc or []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = out + ".tmp%d" % os.getpid()
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


PROBE_LIB = os.path.join(PKG, "libsitu_stream_probe.so")


def build_probe(verbose: bool = False, out: str = PROBE_LIB) -> str:
    """The benchmark's bandwidth probe (csrc/situ_stream_probe.hip), a shared
    library of its own: not part of libsitu_glu.so or its C ABI."""
    tmp = out + ".tmp%d" % os.getpid()
    _run([_hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "situ_stream_probe.hip")], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-q" not in sys.argv))
    print(build_probe(verbose="-q" not in sys.argv))
