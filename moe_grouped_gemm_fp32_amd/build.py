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


def _compile(cmd, out: str, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [tmp if c == out else c for c in cmd]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)
    return out


def build(verbose: bool = True) -> str:
    """Compile libfp8gemm.so next to this file (always rebuilds). Returns its path."""
    return _compile(command(LIB), LIB, verbose)


# Host-sanitizer build: the same library with its host code (argument checks, planner,
# plan cache, workspace and scratch bookkeeping) instrumented by AddressSanitizer and
# UndefinedBehaviorSanitizer, every finding fatal. The device code is built as usual
# (GPU sanitizers are not used). Load it with the sanitizer runtime preloaded
# (sanitizer_runtime()) and FP8GEMM_LIBRARY pointing at it; it is for host-only checks.
LIB_HOSTSAN = os.path.join(PKG, "libfp8gemm_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-g", "-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"]


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of hipcc's clang (for LD_PRELOAD)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or clang
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


def build_host_sanitized(verbose: bool = True, force: bool = False) -> str:
    """Compile libfp8gemm_hostsan.so next to this file unless it is newer than every
    source. Returns its path."""
    srcs = [SRC, *HEADERS, os.path.join(PKG, "csrc", "fp8kgroup_kernel.hpp"),
            os.path.join(PKG, "csrc", "fp8quant_kernel.hpp"), os.path.abspath(__file__)]
    if not force and os.path.exists(LIB_HOSTSAN) and \
            os.path.getmtime(LIB_HOSTSAN) > max(os.path.getmtime(s) for s in srcs):
        return LIB_HOSTSAN
    return _compile(command(LIB_HOSTSAN, extra=HOSTSAN_FLAGS), LIB_HOSTSAN, verbose)


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv[1:]:
        build_host_sanitized(force=True)
    else:
        build()
