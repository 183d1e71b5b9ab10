"""Build libfp8blk.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_scaled_fp8_act_amd.build

Uses hipcc directly; the library lands in block_scaled_fp8_act_amd/lib/.
A second, measurement-only library (libfp8ceil.so: the matrix-core
ceiling kernels that bench.py times beside the GEMM) is built next to it.
fp32 contraction is off (the quantizers' quotient correction relies on
separately rounded multiplies) and packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libfp8blk.so")
SOURCES = ["quant_kernels.hip", "gemm_kernels.hip", "capi.cpp"]
CEIL_LIB = os.path.join(LIBDIR, "libfp8ceil.so")
CEIL_SOURCES = ["ceiling_kernels.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8blk)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    """Build libfp8blk.so (returned) and libfp8ceil.so."""
    path = _build_lib(SOURCES, LIB, verbose)
    _build_lib(CEIL_SOURCES, CEIL_LIB, verbose)
    return path


def _build_lib(sources, lib, verbose: bool) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(), "-c", *lang, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
