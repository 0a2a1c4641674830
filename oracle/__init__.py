"""CPU fp64 oracle for dense C = alpha*A*B + beta*C -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The product path (the HIP library and its Python binding) never
imports it, and the oracle imports nothing from the product path: the two share only the
seeded input generator in ``gemm_inputs``, which holds no GEMM arithmetic.

The arithmetic lives in ``oracle_gemm.c`` (a plain fp64 triple loop, k summed in natural
order, OpenMP over rows); this module only marshals numpy arrays into it. What is computed,
and the pages it follows, is stated at the top of that file:

    C_ref = alpha * (A @ B) + beta * C_in           (fp64, exact fp32 / bf16 / fp16 inputs)
    mag   = |alpha| * (|A| @ |B|) + |beta * C_in|   (elementwise magnitude)

Parity bound (the stated numeric tolerance for fp32 accumulation): an element passes when
``|C_gpu - C_ref| <= REL_TOL * mag``. With alpha = 1 and beta = 0 this is exactly
``1e-5 * sum_k |a_ik * b_kj|``; the alpha/beta extension scales the sum by |alpha| and
adds |beta * c_ij|.

Pins: every function here is checked against values fixed by mathematics rather than by
itself (exact rational brute force, identity and permutation matrices, all-ones, rank-1,
exact integer products, a library fp64 matmul); see ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import build as _build

REL_TOL = 1e-5

_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_lp = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long
_D = ctypes.c_double


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _build.needs_build():
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_num_threads.restype = ctypes.c_int
        full_f32 = [_L, _L, _L, _D, _fp, _L, _fp, _L, _D, _fp, _L, _dp, _dp]
        full_bf16 = [_L, _L, _L, _D, _u16p, _L, _u16p, _L, _D, _fp, _L, _dp, _dp]
        ent_f32 = [_L, _L, _L, _D, _fp, _L, _fp, _L, _D, _fp, _L, _L, _lp, _lp, _dp, _dp]
        ent_bf16 = [_L, _L, _L, _D, _u16p, _L, _u16p, _L, _D, _fp, _L, _L, _lp, _lp, _dp, _dp]
        for name, argt in (("oracle_gemm_f32", full_f32), ("oracle_gemm_bf16", full_bf16),
                           ("oracle_gemm_f16", full_bf16),
                           ("oracle_gemm_f32_entries", ent_f32),
                           ("oracle_gemm_bf16_entries", ent_bf16),
                           ("oracle_gemm_f16_entries", ent_bf16)):
            f = getattr(lib, name)
            f.argtypes = argt
            f.restype = ctypes.c_int
        _lib = lib
        return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct)) if a is not None else ctypes.POINTER(ct)()


def _prep(A, B, C, dtype, M, N, K, b_col_major):
    if dtype == "f32":
        if b_col_major:
            raise ValueError("the fp32 oracle takes row-major B")
        A = np.ascontiguousarray(A, dtype=np.float32).reshape(M, K)
        B = np.ascontiguousarray(B, dtype=np.float32).reshape(K, N)
    elif dtype in ("bf16", "f16"):
        if not b_col_major:
            raise ValueError(f"the {dtype} oracle takes column-major B (stored as N x K)")
        A = np.ascontiguousarray(A, dtype=np.uint16).reshape(M, K)
        B = np.ascontiguousarray(B, dtype=np.uint16).reshape(N, K)
    else:
        raise ValueError(dtype)
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32).reshape(M, N)
    return A, B, C


def gemm(A, B, C=None, *, alpha=1.0, beta=0.0, dtype="f32", b_col_major=None):
    """Full oracle product. A: M x K; B: K x N (fp32, row-major) or N x K storage of a
    column-major K x N bf16 / fp16 matrix (16-bit patterns); C: M x N or None (required when
    beta != 0). Returns (ref, mag) as float64 M x N arrays."""
    if b_col_major is None:
        b_col_major = dtype in ("bf16", "f16")
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    N = B.shape[0] if b_col_major else B.shape[1]
    if (B.shape[1] if b_col_major else B.shape[0]) != K:
        raise ValueError("inner dimensions differ")
    if beta != 0.0 and C is None:
        raise ValueError("beta != 0 needs C")
    A, B, C = _prep(A, B, C if beta != 0.0 else None, dtype, M, N, K, b_col_major)
    out = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    lib = _load()
    if dtype == "f32":
        rc = lib.oracle_gemm_f32(M, N, K, float(alpha), _ptr(A, ctypes.c_float), K,
                                 _ptr(B, ctypes.c_float), N, float(beta),
                                 _ptr(C, ctypes.c_float), N, _ptr(out, ctypes.c_double),
                                 _ptr(mag, ctypes.c_double))
    else:
        fn = lib.oracle_gemm_bf16 if dtype == "bf16" else lib.oracle_gemm_f16
        rc = fn(M, N, K, float(alpha), _ptr(A, ctypes.c_uint16), K,
                _ptr(B, ctypes.c_uint16), K, float(beta),
                _ptr(C, ctypes.c_float), N, _ptr(out, ctypes.c_double),
                _ptr(mag, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return out, mag


def gemm_entries(A, B, C, I, J, *, alpha=1.0, beta=0.0, dtype="f32", b_col_major=None):
    """Oracle values at the sampled positions (I[e], J[e]); returns (ref, mag) of length n."""
    if b_col_major is None:
        b_col_major = dtype in ("bf16", "f16")
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    N = B.shape[0] if b_col_major else B.shape[1]
    if beta != 0.0 and C is None:
        raise ValueError("beta != 0 needs C")
    A, B, C = _prep(A, B, C if beta != 0.0 else None, dtype, M, N, K, b_col_major)
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D and equally long")
    n = I.shape[0]
    out = np.empty(n, np.float64)
    mag = np.empty(n, np.float64)
    lib = _load()
    fn = {"f32": lib.oracle_gemm_f32_entries, "bf16": lib.oracle_gemm_bf16_entries,
          "f16": lib.oracle_gemm_f16_entries}[dtype]
    ct = ctypes.c_float if dtype == "f32" else ctypes.c_uint16
    rc = fn(M, N, K, float(alpha), _ptr(A, ct), K, _ptr(B, ct), K if b_col_major else N,
            float(beta), _ptr(C, ctypes.c_float), N, n, _ptr(I, ctypes.c_long),
            _ptr(J, ctypes.c_long), _ptr(out, ctypes.c_double), _ptr(mag, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return out, mag


def gemm_inputs(inp):
    """Oracle on a ``gemm_inputs.GemmInputs`` problem."""
    return gemm(inp.A, inp.B, inp.C, alpha=inp.alpha, beta=inp.beta, dtype=inp.dtype,
                b_col_major=inp.b_col_major)


def gemm_inputs_entries(inp, I, J):
    return gemm_entries(inp.A, inp.B, inp.C, I, J, alpha=inp.alpha, beta=inp.beta,
                        dtype=inp.dtype, b_col_major=inp.b_col_major)


def bound(mag):
    """Per-element parity bound REL_TOL * mag."""
    return REL_TOL * np.asarray(mag, dtype=np.float64)


def check(got, ref, mag):
    """Return (ok, worst_ratio) where ratio = |got - ref| / bound (non-finite got fails)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    b = bound(mag)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0, err / b, np.where(err == 0, 0.0, np.inf))
    ratio = np.where(np.isfinite(got), ratio, np.inf)
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst
