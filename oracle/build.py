"""Compile the CPU oracle library (test infrastructure only; see dd_gemm_oracle.c)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dd_gemm_oracle.c")
LIB = os.path.join(HERE, "libddoracle.so")

CFLAGS = [
    "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
    "-march=x86-64-v3",          # AVX2 + FMA: fma() is one fused instruction
    "-ffp-contract=off",         # no implicit fusion of a*b+c
    "-fno-fast-math",
]


def build(verbose: bool = True) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
