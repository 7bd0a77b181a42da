"""Builds libsbn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsbn.so")

SOURCES = ["api.hip", "quantize_act.hip", "pack.hip", "bitlinear.hip", "backward.hip",
           "outliers.hip", "gemv_i8.hip", "gemv_bf16.hip", "ceilings.hip", "static_ws.hip"]
HEADERS = ["sbn_common.hpp", "sbn_internal.hpp", "gemv.hpp"]
# The int8-input GEMV entries and the one-token bf16 entry take their first loads' operands as
# leading scalar arguments, which the firmware preloads into registers with this option.
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
EXTRA_FLAGS = {"gemv_i8.hip": _PRELOAD, "gemv_bf16.hip": _PRELOAD}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed fp32 VALU ops stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                     and "warning: feature flag" not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compiles every source (always; no staleness check) and links libsbn.so."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
