"""Build libddgemm.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libddgemm.so")
SOURCES = ["api.cpp", "split_k.cpp", "split.hip", "qd_split.hip", "sliced_gemm.hip", "levels.hip", "accumulate.hip",
           "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                       # error-free transformations must not be fused
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = True, extra_flags=()) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if msgs and (verbose or res.returncode != 0):
        print("\n".join(msgs), file=sys.stderr, flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
