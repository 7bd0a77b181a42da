"""Builds libsbn_san.so: the library with its host code (the C ABI's argument validation and handle
lifecycle, api.hip, static_ws.hip and ceilings.hip) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer, for running the boundary tests on the CPU. The kernel sources are
linked from the regular build's objects. GPU code is never built with a sanitizer: every
-fsanitize= applies to the host pass only.

Load it with the sanitizer runtime preloaded, e.g.
  LD_PRELOAD=$(python -m sparsity_sbn_quantize_amd.build_sanitized --runtime) \\
  SBN_LIB=sparsity_sbn_quantize_amd/_build/san/libsbn_san.so python -m pytest tests/test_abi_cpu.py
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

from sparsity_sbn_quantize_amd import build as B

SAN_SOURCES = ["api.hip", "static_ws.hip", "ceilings.hip"]
SAN_BUILD = os.path.join(B.BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libsbn_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]
CLANG = "/opt/rocm/llvm/bin/clang++"


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime that must be preloaded into the host process."""
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not libs:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return sorted(libs)[-1]


def build_sanitized() -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    if not all(os.path.exists(os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o"))
               for s in B.SOURCES):
        B.build(verbose=False)
    objs = []
    for src in SAN_SOURCES:
        obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [B.HIPCC, *B.FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile failed for {src}:\n{r.stderr}")
        objs.append(obj)
    objs += [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
             if s not in SAN_SOURCES]
    san = ["-fsanitize=" + k for k in ("address", "undefined")]
    cmd = [CLANG, "-shared", "-fPIC", *san, "-shared-libasan", "-o", SAN_LIB, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if "--runtime" in sys.argv:
        print(runtime())
    else:
        print(build_sanitized())
