"""The C ABI's host code (argument validation, the handle and workspace entry points) built with
AddressSanitizer and UndefinedBehaviorSanitizer runs the boundary tests clean on the CPU. The
kernels are not instrumented (GPU code is never built with a sanitizer); no GPU is needed."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="needs hipcc")
def test_boundary_tests_under_host_sanitizers():
    from sparsity_sbn_quantize_amd import build_sanitized as S
    lib = S.build_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "host code not instrumented"
    env = dict(os.environ, LD_PRELOAD=S.runtime(), SBN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m",
                        "not gpu", "tests/test_abi_cpu.py", "tests/test_zz_no_alloc.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr
