"""Blocked multithreaded fp32 CPU GEMM -- a performance baseline for bench.py only.

Not the correctness reference (that is ``oracle/``) and not part of the product path: the HIP
library never calls it. ``blocked_gemm.c`` holds the arithmetic; this module builds it with gcc
(-O3 -mavx2 -mfma -fopenmp) and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "blocked_gemm.c")
LIB = os.path.join(HERE, "libblocked.so")
_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O3", "-std=gnu11", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", SRC,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        L, F, P = ctypes.c_long, ctypes.c_float, ctypes.c_void_p
        lib.blocked_sgemm.argtypes = [L, L, L, F, P, L, P, L, F, P, L]
        lib.blocked_sgemm.restype = ctypes.c_int
        lib.blocked_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().blocked_num_threads())


def sgemm(A, B, C=None, alpha=1.0, beta=0.0):
    """C = alpha*A@B + beta*C in fp32 on the host (row-major float32 arrays); returns C."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if C is None:
        C = np.zeros((M, N), np.float32)
    C = np.ascontiguousarray(C, dtype=np.float32)
    rc = _load().blocked_sgemm(M, N, K, float(alpha), A.ctypes.data, K, B.ctypes.data, N,
                               float(beta), C.ctypes.data, N)
    if rc != 0:
        raise RuntimeError(f"blocked_sgemm failed ({rc})")
    return C
