"""Seeded synthetic GEMM inputs, shared by the CPU oracle tests and the HIP-path tests.

This module only draws matrices and encodes fp32 draws as bf16 or fp16 bit patterns. It holds
none of the product's arithmetic: no sums, no products, no tiling. Both sides of every
parity check (the fp64 oracle under ``oracle/`` and the HIP library) receive the very
same host arrays from here.

Draw order and layout
---------------------
* ``numpy.random.Generator(PCG64(seed))``; one generator per workload.
* The buffers are drawn in the order A, then B, then C_in, each as one flat array in
  its storage order (row-major A and C; B row-major for the fp32 workloads, column-major
  for the bf16 workload, i.e. stored as N rows of K values).
* ``uniform`` is ``rng.uniform(-1, 1).astype(float32)``; ``normal`` is
  ``rng.standard_normal(dtype=float32)``.
* bf16 operands are the round-to-nearest-even encoding of the fp32 draw (NaN becomes the
  quiet NaN 0x7FC0). The pages fix no rounding mode; this is the plain reading.
* fp16 operands (the pages' worked half-precision GEMM) are numpy's float32 -> float16
  conversion of the draw: IEEE binary16, round to nearest even, overflow to infinity.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "f32_to_f16_bits",
    "draw",
    "GemmInputs",
    "make_inputs",
]


@dataclass(frozen=True)
class Workload:
    """One GEMM workload: shape, dtype, layout, value distribution, alpha/beta, seed."""

    name: str
    M: int
    N: int
    K: int
    dtype: str  # "f32" (fp32 in, fp32 out), "bf16" or "f16" (16-bit in, fp32 out)
    dist: str  # "uniform" (U[-1,1]) or "normal" (N(0,1))
    alpha: float = 1.0
    beta: float = 0.0
    seed: int = 0
    b_col_major: bool = False
    description: str = ""

    @property
    def flop(self) -> int:
        """Algorithmic work of the product: 2*M*N*K (the 3*M*N epilogue flops excluded)."""
        return 2 * self.M * self.N * self.K


# The five workloads: a small correctness case, the square fp32 case, a ragged case
# with a non-trivial epilogue, the square bf16 case (column-major B) and a tall-skinny case;
# then fp16 operands at the bf16 case's shape, the fp32 path at that shape, and a bf16 problem of
# few output tiles with a deep K.
WORKLOADS = {
    "f32_256": Workload("f32_256", 256, 256, 256, "f32", "uniform", 1.0, 0.0, 1001,
                        description="fp32 256^3, U[-1,1], alpha=1, beta=0"),
    "f32_4096": Workload("f32_4096", 4096, 4096, 4096, "f32", "uniform", 1.0, 0.0, 1002,
                         description="fp32 4096^3, U[-1,1], alpha=1, beta=0"),
    "f32_ragged": Workload("f32_ragged", 1000, 1500, 777, "f32", "normal", 1.5, -0.5, 1003,
                           description="fp32 M=1000 N=1500 K=777, N(0,1), alpha=1.5, beta=-0.5, C_in N(0,1)"),
    "bf16_8192": Workload("bf16_8192", 8192, 8192, 8192, "bf16", "normal", 1.0, 0.0, 1004,
                          b_col_major=True,
                          description="bf16 8192^3, A row-major, B column-major, N(0,1) rounded to bf16, fp32 C"),
    "f32_tall": Workload("f32_tall", 16384, 128, 4096, "f32", "uniform", 1.0, 0.0, 1005,
                         description="fp32 tall-skinny M=16384 N=128 K=4096, U[-1,1], alpha=1, beta=0"),
    "f16_8192": Workload("f16_8192", 8192, 8192, 8192, "f16", "normal", 1.0, 0.0, 1006,
                         b_col_major=True,
                         description="fp16 8192^3, A row-major, B column-major, N(0,1) rounded to fp16, fp32 C"),
    "f32_8192": Workload("f32_8192", 8192, 8192, 8192, "f32", "uniform", 1.0, 0.0, 1007,
                         description="fp32 8192^3, U[-1,1], alpha=1, beta=0 (the fp32 path at the bf16 size)"),
    "bf16_few": Workload("bf16_few", 1024, 1024, 16384, "bf16", "normal", 1.0, 0.0, 1008,
                         b_col_major=True,
                         description="bf16 M=N=1024 K=16384 (few output tiles), A row-major, B column-major, "
                                     "N(0,1) rounded to bf16, fp32 C"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even); uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(rng: np.random.Generator, n: int, dist: str) -> np.ndarray:
    """n float32 values from the named distribution."""
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, n).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(n, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


@dataclass
class GemmInputs:
    """Host buffers of one GEMM problem in the library's storage layout.

    A: M x K row-major (lda = K). B: K x N row-major (ldb = N), or for ``b_col_major``
    K x N column-major, stored as an N x K array (ldb = K). C: M x N row-major (ldc = N),
    present only when beta != 0. For bf16 and fp16 workloads A and B hold uint16 bit patterns.
    """

    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dtype: str
    b_col_major: bool
    A: np.ndarray
    B: np.ndarray
    C: Optional[np.ndarray] = field(default=None)

    @property
    def lda(self) -> int:
        return self.A.shape[1] if self.A.ndim == 2 else self.K

    @property
    def ldb(self) -> int:
        return self.B.shape[1] if self.B.ndim == 2 else (self.K if self.b_col_major else self.N)

    @property
    def ldc(self) -> int:
        return self.N


def make_inputs(M: int, N: int, K: int, *, dtype: str = "f32", dist: str = "uniform",
                alpha: float = 1.0, beta: float = 0.0, seed: int = 0,
                b_col_major: Optional[bool] = None, with_c: Optional[bool] = None) -> GemmInputs:
    """Draw one problem. ``b_col_major`` defaults to True for bf16 / fp16 and False for fp32;
    C_in is drawn (same distribution) when beta != 0 or ``with_c`` is set."""
    if b_col_major is None:
        b_col_major = dtype in ("bf16", "f16")
    if with_c is None:
        with_c = beta != 0.0
    rng = np.random.Generator(np.random.PCG64(seed))
    a = draw(rng, M * K, dist).reshape(M, K)
    if b_col_major:
        b = draw(rng, K * N, dist).reshape(N, K)
    else:
        b = draw(rng, K * N, dist).reshape(K, N)
    c = draw(rng, M * N, dist).reshape(M, N) if with_c else None
    if dtype == "bf16":
        a = f32_to_bf16_bits(a).reshape(a.shape)
        b = f32_to_bf16_bits(b).reshape(b.shape)
    elif dtype == "f16":
        a = f32_to_f16_bits(a).reshape(a.shape)
        b = f32_to_f16_bits(b).reshape(b.shape)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return GemmInputs(M, N, K, float(alpha), float(beta), dtype, bool(b_col_major), a, b, c)


def workload_inputs(w: Workload) -> GemmInputs:
    return make_inputs(w.M, w.N, w.K, dtype=w.dtype, dist=w.dist, alpha=w.alpha, beta=w.beta,
                       seed=w.seed, b_col_major=w.b_col_major)


__all__.append("workload_inputs")
