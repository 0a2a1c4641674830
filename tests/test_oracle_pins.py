"""Pins of the fp64 CPU oracle against values fixed by mathematics, not by the oracle itself.

Each pin is chosen so that a plausible slip in the oracle -- a dropped k term, a wrong
sign, a swapped index, a transposed operand, a wrong alpha/beta convention, a wrong bf16
widening or a wrong column-major stride -- fails at least one test:

* exact rational brute force (``fractions.Fraction``) on every shape with M, N, K in 1..5;
* identity and permutation matrices (result equals the other operand, bitwise);
* all-ones (every entry equals K exactly) and rank-1 outer products;
* integer-valued matrices against exact int64 products (non-square, so a transposition
  cannot pass);
* a library fp64 matmul within the fp64 summation error bound;
* the BLAS alpha/beta conventions (beta == 0 never reads C, alpha == 0 never reads A, B);
* bf16 bit patterns whose values follow from the format's definition.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle

U53 = 2.0 ** -53


def _frac_f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def _widen_bf16_independent(h: int) -> float:
    """bf16 bits -> value via the byte layout of an IEEE binary32 word (independent of both
    the generator and the oracle)."""
    return struct.unpack(">f", struct.pack(">I", (int(h) & 0xFFFF) << 16))[0]


def _widen_f16_independent(h: int) -> float:
    """fp16 bits -> value via Python's own IEEE binary16 unpacking (struct format 'e')."""
    return struct.unpack("<e", struct.pack("<H", int(h) & 0xFFFF))[0]


def _exact_gemm(A, B, C, alpha, beta, dtype, b_col_major):
    """alpha*A*B + beta*C and |alpha|*|A||B| + |beta C| in exact rationals."""
    M, K = A.shape
    N = B.shape[0] if b_col_major else B.shape[1]
    if dtype in ("bf16", "f16"):
        w = _widen_bf16_independent if dtype == "bf16" else _widen_f16_independent
        fa = [[Fraction(w(A[i, k])) for k in range(K)] for i in range(M)]
        fb = [[Fraction(w(B[j, k] if b_col_major else B[k, j]))
               for j in range(N)] for k in range(K)]
    else:
        fa = [[_frac_f32(A[i, k]) for k in range(K)] for i in range(M)]
        fb = [[_frac_f32(B[k, j]) for j in range(N)] for k in range(K)]
    al, be = Fraction(alpha), Fraction(beta)
    ref = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = sum((fa[i][k] * fb[k][j] for k in range(K)), Fraction(0))
            t = sum((abs(fa[i][k] * fb[k][j]) for k in range(K)), Fraction(0))
            c = _frac_f32(C[i, j]) if beta != 0.0 else Fraction(0)
            ref[i][j] = al * s + be * c
            mag[i][j] = abs(al) * t + abs(be * c)
    return ref, mag


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_bruteforce_every_tiny_shape(dtype):
    rng = np.random.Generator(np.random.PCG64(7))
    alphas = [1.0, -0.5, 1.5, 0.0, 3.0]
    betas = [0.0, -0.5, 1.0, 2.25]
    case = 0
    for M in range(1, 6):
        for N in range(1, 6):
            for K in range(1, 6):
                alpha = alphas[case % len(alphas)]
                beta = betas[(case // 3) % len(betas)]
                case += 1
                inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=alpha,
                                     beta=beta, seed=int(rng.integers(1 << 30)))
                ref, mag = oracle.gemm_inputs(inp)
                ex_ref, ex_mag = _exact_gemm(inp.A, inp.B, inp.C, alpha, beta, dtype,
                                             inp.b_col_major)
                for i in range(M):
                    for j in range(N):
                        err = abs(Fraction(float(ref[i, j])) - ex_ref[i][j])
                        # fp64 recursive summation of K exact products, then alpha*s, beta*c, +.
                        lim = Fraction((K + 3) * U53) * ex_mag[i][j]
                        assert err <= lim, (dtype, M, N, K, i, j, float(err), float(lim))
                        merr = abs(Fraction(float(mag[i, j])) - ex_mag[i][j])
                        assert merr <= Fraction((K + 3) * U53) * ex_mag[i][j]


def test_bruteforce_random_small_shapes():
    rng = np.random.Generator(np.random.PCG64(11))
    for t in range(12):
        M, N, K = (int(v) for v in rng.integers(1, 13, 3))
        inp = gi.make_inputs(M, N, K, dtype="f32", dist="uniform", alpha=1.25, beta=-0.75,
                             seed=100 + t)
        ref, mag = oracle.gemm_inputs(inp)
        ex_ref, ex_mag = _exact_gemm(inp.A, inp.B, inp.C, 1.25, -0.75, "f32", False)
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(float(ref[i, j])) - ex_ref[i][j])
                assert err <= Fraction((K + 3) * U53) * ex_mag[i][j]


def test_identity_left_and_right():
    rng = np.random.Generator(np.random.PCG64(3))
    n, m = 37, 53
    B = rng.standard_normal((n, m), dtype=np.float32)
    ref, _ = oracle.gemm(np.eye(n, dtype=np.float32), B)
    assert np.array_equal(ref, B.astype(np.float64))
    A = rng.standard_normal((m, n), dtype=np.float32)
    ref, _ = oracle.gemm(A, np.eye(n, dtype=np.float32))
    assert np.array_equal(ref, A.astype(np.float64))


def test_permutation_reorders_rows_and_columns():
    rng = np.random.Generator(np.random.PCG64(4))
    n, m = 29, 17
    perm = rng.permutation(n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), perm] = 1.0
    B = rng.standard_normal((n, m), dtype=np.float32)
    ref, _ = oracle.gemm(P, B)  # (P B)[i] = B[perm[i]]
    assert np.array_equal(ref, B[perm].astype(np.float64))
    A = rng.standard_normal((m, n), dtype=np.float32)
    ref, _ = oracle.gemm(A, P)  # (A P)[:, perm[i]] = A[:, i]
    expect = np.empty_like(A)
    expect[:, perm] = A
    assert np.array_equal(ref, expect.astype(np.float64))


@pytest.mark.parametrize("K", [1, 7, 256, 4097])
def test_all_ones_gives_K(K):
    A = np.ones((5, K), np.float32)
    B = np.ones((K, 9), np.float32)
    ref, mag = oracle.gemm(A, B)
    assert np.all(ref == K) and np.all(mag == K)
    ref, _ = oracle.gemm(A, B, alpha=0.25)
    assert np.all(ref == K * 0.25)
    hb = np.full((9, K), 0x3F80, np.uint16)  # bf16 1.0, column-major B
    ha = np.full((5, K), 0x3F80, np.uint16)
    ref, mag = oracle.gemm(ha, hb, dtype="bf16")
    assert np.all(ref == K) and np.all(mag == K)


def test_rank1_outer_products():
    rng = np.random.Generator(np.random.PCG64(5))
    u = rng.standard_normal(31, dtype=np.float32)
    v = rng.standard_normal(23, dtype=np.float32)
    ref, _ = oracle.gemm(u[:, None], v[None, :])
    # a product of two fp32 numbers is exact in fp64
    for i in (0, 7, 30):
        for j in (0, 11, 22):
            assert Fraction(float(ref[i, j])) == _frac_f32(u[i]) * _frac_f32(v[j])
    # K > 1 with integer columns: C = K * u v^T exactly
    ui = rng.integers(-9, 10, 31).astype(np.float32)
    vi = rng.integers(-9, 10, 23).astype(np.float32)
    K = 40
    ref, _ = oracle.gemm(np.repeat(ui[:, None], K, 1), np.repeat(vi[None, :], K, 0))
    assert np.array_equal(ref, K * np.outer(ui.astype(np.int64), vi.astype(np.int64)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 200, 17), (129, 67, 300), (64, 130, 1000)])
def test_integer_matrices_exact_f32(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 1000 + N + K))
    Ai = rng.integers(-16, 17, (M, K))
    Bi = rng.integers(-16, 17, (K, N))
    Ci = rng.integers(-16, 17, (M, N))
    ref, mag = oracle.gemm(Ai.astype(np.float32), Bi.astype(np.float32),
                           Ci.astype(np.float32), alpha=2.0, beta=-3.0)
    assert np.array_equal(ref, 2 * (Ai @ Bi) - 3 * Ci)
    assert np.array_equal(mag, 2 * (np.abs(Ai) @ np.abs(Bi)) + 3 * np.abs(Ci))


@pytest.mark.parametrize("M,N,K", [(5, 3, 2), (70, 33, 129), (31, 260, 400)])
def test_integer_matrices_exact_bf16_column_major(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M + 17 * N + K))
    Ai = rng.integers(-16, 17, (M, K))
    Bi = rng.integers(-16, 17, (K, N))
    ha = gi.f32_to_bf16_bits(Ai.astype(np.float32)).reshape(M, K)
    hbT = gi.f32_to_bf16_bits(np.ascontiguousarray(Bi.T).astype(np.float32)).reshape(N, K)
    ref, mag = oracle.gemm(ha, hbT, dtype="bf16")
    assert np.array_equal(ref, Ai @ Bi)
    assert np.array_equal(mag, np.abs(Ai) @ np.abs(Bi))


@pytest.mark.parametrize("M,N,K", [(5, 3, 2), (70, 33, 129), (31, 260, 400)])
def test_integer_matrices_exact_f16_column_major(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 1000 + N + K))
    Ai = rng.integers(-16, 17, (M, K))
    Bi = rng.integers(-16, 17, (K, N))
    ha = gi.f32_to_f16_bits(Ai.astype(np.float32)).reshape(M, K)
    hbT = gi.f32_to_f16_bits(np.ascontiguousarray(Bi.T).astype(np.float32)).reshape(N, K)
    ref, mag = oracle.gemm(ha, hbT, dtype="f16")
    assert np.array_equal(ref, (Ai @ Bi).astype(np.float64))
    assert np.array_equal(mag, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def test_against_library_fp64_matmul():
    rng = np.random.Generator(np.random.PCG64(12))
    M, N, K = 257, 129, 300
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.standard_normal((M, N), dtype=np.float32)
    ref, mag = oracle.gemm(A, B, C, alpha=1.5, beta=-0.5)
    lib = 1.5 * (A.astype(np.float64) @ B.astype(np.float64)) - 0.5 * C.astype(np.float64)
    # both sides carry fp64 rounding: allow twice the summation bound
    assert np.all(np.abs(ref - lib) <= 2 * (K + 3) * U53 * mag)
    lib_mag = 1.5 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)) \
        + 0.5 * np.abs(C.astype(np.float64))
    assert np.allclose(mag, lib_mag, rtol=4 * (K + 3) * U53, atol=0)


def test_blas_alpha_beta_conventions():
    rng = np.random.Generator(np.random.PCG64(13))
    M, N, K = 9, 11, 13
    A = rng.standard_normal((M, K), dtype=np.float32)
    B = rng.standard_normal((K, N), dtype=np.float32)
    Cnan = np.full((M, N), np.nan, np.float32)
    ref, mag = oracle.gemm(A, B, Cnan, beta=0.0)  # beta == 0: C is never read
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(mag))
    C = rng.standard_normal((M, N), dtype=np.float32)
    Anan = np.full((M, K), np.nan, np.float32)
    ref, mag = oracle.gemm(Anan, B, C, alpha=0.0, beta=-0.5)  # alpha == 0: A, B not read
    assert np.array_equal(ref, -0.5 * C.astype(np.float64))
    assert np.array_equal(mag, 0.5 * np.abs(C.astype(np.float64)))
    # K == 0: C = beta * C
    ref, _ = oracle.gemm(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), C,
                         beta=2.0)
    assert np.array_equal(ref, 2.0 * C.astype(np.float64))
    # power-of-two alpha scales exactly
    r1, _ = oracle.gemm(A, B)
    r8, _ = oracle.gemm(A, B, alpha=8.0)
    assert np.array_equal(r8, 8.0 * r1)
    # a sign slip in beta would fail this
    rb, _ = oracle.gemm(A, B, C, alpha=1.0, beta=-1.0)
    assert np.array_equal(rb, r1 - C.astype(np.float64))


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5), (0x4049, 3.140625),
    (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126), (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127),
    (0xC2F7, -123.5), (0x0000, 0.0), (0x8000, -0.0), (0x7F80, float("inf")),
])
def test_bf16_widening_follows_the_format(bits, value):
    # bf16 = sign, 8-bit exponent (bias 127), 7 fraction bits: value read off the definition
    one = np.array([[0x3F80]], np.uint16)
    ref, _ = oracle.gemm(np.array([[bits]], np.uint16), one, dtype="bf16")
    # (a zero product added to the +0.0 start of the sum is +0.0, so only the value is compared)
    assert ref[0, 0] == value


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xBC00, -1.0), (0x4000, 2.0), (0x3800, 0.5), (0x4248, 3.140625),
    (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14), (0x7BFF, 65504.0),
    (0xD7B8, -123.5), (0x0000, 0.0), (0x8000, -0.0), (0x7C00, float("inf")),
])
def test_f16_widening_follows_the_format(bits, value):
    # IEEE binary16 = sign, 5-bit exponent (bias 15), 10 fraction bits; exponent 0 holds the
    # subnormals f * 2^-24: value read off the definition
    one = np.array([[0x3C00]], np.uint16)
    ref, _ = oracle.gemm(np.array([[bits]], np.uint16), one, dtype="f16")
    assert ref[0, 0] == value


def test_sampled_entries_match_full_product():
    for dtype in ("f32", "bf16", "f16"):
        inp = gi.make_inputs(67, 45, 129, dtype=dtype, dist="normal", alpha=1.5, beta=-0.5,
                             seed=21)
        ref, mag = oracle.gemm_inputs(inp)
        rng = np.random.Generator(np.random.PCG64(22))
        I = rng.integers(0, 67, 300)
        J = rng.integers(0, 45, 300)
        er, em = oracle.gemm_inputs_entries(inp, I, J)
        assert np.array_equal(er, ref[I, J]) and np.array_equal(em, mag[I, J])


def test_sampled_entries_reject_out_of_range():
    inp = gi.make_inputs(4, 4, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm_inputs_entries(inp, [0, 4], [0, 0])


def test_check_and_bound():
    ref = np.array([1.0, 2.0, 0.0])
    mag = np.array([1.0, 10.0, 0.0])
    ok, worst = oracle.check(np.array([1.0 + 1e-6, 2.0 - 5e-5, 0.0]), ref, mag)
    assert ok and abs(worst - 1.0) < 1e-9 or worst <= 1.0
    ok, worst = oracle.check(np.array([1.0 + 2e-5, 2.0, 0.0]), ref, mag)
    assert not ok and worst > 1.9
    ok, _ = oracle.check(np.array([1.0, 2.0, 1e-30]), ref, mag)  # zero bound, nonzero error
    assert not ok
    ok, _ = oracle.check(np.array([np.nan, 2.0, 0.0]), ref, mag)
    assert not ok
