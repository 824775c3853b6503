"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
host-side suites (argument validation, planner invariants, plan cache, the measured
plan table) run in a child process against the host-sanitizer build, with the
sanitizer runtime preloaded. Any finding aborts the child. No GPU is used: these
suites never launch a kernel."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_host.py", "tests/test_planner_table.py"]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the host-sanitizer library")
def test_host_suites_under_address_and_undefined_behavior_sanitizers():
    from moe_grouped_gemm_fp32_amd import build  # the build helpers, imported only here

    lib = build.build_host_sanitized(verbose=False)
    runtime = build.sanitizer_runtime()
    nm = shutil.which("nm")
    if nm:  # the build really is instrumented: it calls into both sanitizer runtimes
        syms = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, FP8GEMM_LIBRARY=lib,
               # leaks of the interpreter itself are not the library's; every other finding aborts
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          *SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in res.stdout
