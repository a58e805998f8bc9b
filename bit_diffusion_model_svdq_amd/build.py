"""Builds libsvdq.so in-tree: HIP sources with hipcc for gfx950, the host packer with g++.

Run as ``python bit_diffusion_model_svdq_amd/build.py`` (by path: importing the package
needs the library).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvdq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    # packed fp32 VALU forms stay disabled: plain float ops only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fopenmp",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]

HIP_SOURCES = ["svdq_api.hip", "k1_smooth_quant.hip", "k2_w4a4_gemm.hip", "k2_mxfp4_gemm.hip",
               "calib_absmax.hip", "k12_fused_smallk.hip"]
CXX_SOURCES = ["pack.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    return r


# Host sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for the host
# code only: the packer and the entry points' argument checks.  Device code is
# built as usual; every -fsanitize= on a hipcc line sits behind -Xarch_host.
# One runtime serves the whole library (clang's shared one), so the packer is
# compiled with ROCm's clang++ rather than g++ here.
SAN = ["-fsanitize=address", "-fsanitize=undefined"]
SAN_LIB = os.path.join(PKG, "_build", "san", "libsvdq_san.so")


def build_sanitized(verbose: bool = False) -> str:
    """libsvdq with ASan/UBSan on its host code (a test build, not the product).
    Load it with SVDQ_LIBRARY=<path> and the sanitizer runtime preloaded."""
    out = os.path.dirname(SAN_LIB)
    os.makedirs(out, exist_ok=True)
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    common = ["-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(out, src + ".o")
        flags = [f if f != "-O3" else "-O1" for f in HIP_FLAGS]
        _run([HIPCC, *flags, *host_san, *[a for f in common for a in ("-Xarch_host", f)], "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    clangxx = os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang++")
    for src in CXX_SOURCES:
        obj = os.path.join(out, src + ".o")
        flags = [f if f != "-O3" else "-O1" for f in CXX_FLAGS]
        _run([clangxx, *flags, *SAN, *common, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fopenmp", "-shared-libsan",
          *host_san, *objs, "-o", SAN_LIB])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        _run([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fopenmp", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
