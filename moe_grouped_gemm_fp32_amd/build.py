"""Ahead-of-time build of libfp8gemm.so for gfx950 (hipcc, in-tree).

Every kernel variant is a template instance compiled once here; the host code
picks one per call. Packed-FP32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fp8gemm.hip")
HEADERS = [os.path.join(PKG, "csrc", "fp8gemm_kernel.hpp"), os.path.join(ROOT, "include", "fp8gemm.h")]
LIB = os.path.join(PKG, "libfp8gemm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def command(out: str, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the FP32 promotion FMAs read them directly
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), *extra, SRC, "-o", out]


def build(verbose: bool = True) -> str:
    """Compile libfp8gemm.so next to this file (always rebuilds). Returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp8gemm.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
