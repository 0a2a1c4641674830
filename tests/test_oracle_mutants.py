"""The oracle pins are strong enough: each planted slip in a copy of the oracle's C source
(compiled on the CPU into a temporary library) must make at least one pin fail.

Mutations stay in bounds (they change which in-range element is read or how it is
combined), so every mutant runs to completion and only its values differ.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild

import test_oracle_pins as pins

MUTANTS = {
    "drop_last_k_term_f32": ("for (long k = 0; k < K; ++k) {\n                double a",
                             "for (long k = 0; k + 1 < K; ++k) {\n                double a"),
    "subtract_products_f32": ("o[j] += p;", "o[j] -= p;"),
    "mirror_b_column_f32": ("double p = a * (double)brow[j];",
                            "double p = a * (double)brow[N - 1 - j];"),
    "beta_ignored_f32": ("o[j] = alpha * o[j] + bc;", "o[j] = alpha * o[j];"),
    "alpha_ignored_f32": ("o[j] = alpha * o[j] + bc;", "o[j] = o[j] + bc;"),
    "c_read_transposed_f32": ("double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;\n            o[j]",
                              "double bc = (beta != 0.0) ? beta * (double)C[(i % N) * ldc + (j % M)] : 0.0;\n            o[j]"),
    "widen_shift_wrong": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "bf16_b_row_stride": ("const uint16_t *bcol = B + j * ldb;\n                for",
                          "const uint16_t *bcol = B + (N - 1 - j) * ldb;\n                for"),
    "bf16_drop_first_k": ("for (long k = 0; k < K; ++k) {\n                    double p = widen_bf16(arow[k])",
                          "for (long k = 1; k < K; ++k) {\n                    double p = widen_bf16(arow[k])"),
    "mag_without_abs": ("g[j] += fabs(p);", "g[j] += p;"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "f16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "f16_fraction_width": ("int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;",
                           "int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x1FF;"),
}

PIN_TESTS = [
    lambda: pins.test_bruteforce_every_tiny_shape("f32"),
    lambda: pins.test_bruteforce_every_tiny_shape("bf16"),
    lambda: pins.test_integer_matrices_exact_f32(129, 67, 300),
    lambda: pins.test_integer_matrices_exact_bf16_column_major(70, 33, 129),
    pins.test_blas_alpha_beta_conventions,
    pins.test_identity_left_and_right,
    pins.test_permutation_reorders_rows_and_columns,
    lambda: pins.test_bf16_widening_follows_the_format(0x4049, 3.140625),
    lambda: pins.test_bruteforce_every_tiny_shape("f16"),
    lambda: pins.test_integer_matrices_exact_f16_column_major(70, 33, 129),
    lambda: pins.test_f16_widening_follows_the_format(0x0001, 2.0 ** -24),
    lambda: pins.test_f16_widening_follows_the_format(0x4248, 3.140625),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", str(c), "-o", str(so), "-lm"], check=True)
    return str(so)


def _configure(lib):
    real = oracle._load()
    for fname in ("oracle_gemm_f32", "oracle_gemm_bf16", "oracle_gemm_f16", "oracle_gemm_f32_entries",
                  "oracle_gemm_bf16_entries", "oracle_gemm_f16_entries", "oracle_num_threads"):
        f = getattr(lib, fname)
        g = getattr(real, fname)
        f.argtypes = g.argtypes
        f.restype = g.restype
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    lib = _configure(ctypes.CDLL(_build_mutant(tmp_path, name, old, new)))
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    lib = _configure(ctypes.CDLL(_build_mutant(tmp_path, "none", "int oracle_num_threads",
                                               "int oracle_num_threads")))
    monkeypatch.setattr(oracle, "_lib", lib)
    for t in PIN_TESTS:
        t()
