"""Builds the CPU oracle library ``oracle/liboracle.so`` with gcc (test infrastructure only).

Plain optimisation (-O2), no fast-math and no FMA contraction, OpenMP over output rows.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def needs_build() -> bool:
    return not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
