"""The seeded generator: determinism, layouts, and bf16 round-to-nearest-even against two
independent encoders (exact rational nearest-with-ties-to-even, and torch's CPU cast)."""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs as gi


def _bf16_rne_exact(x: float) -> int:
    """Nearest bf16 to x by exact comparison, ties to an even fraction field."""
    bits = struct.unpack(">I", struct.pack(">f", x))[0]
    if (bits & 0x7F800000) == 0x7F800000:
        return 0x7FC0 if (bits & 0x7FFFFF) else bits >> 16  # NaN, or +-infinity kept
    lo = bits >> 16  # truncation toward zero
    hi = lo + 1  # next bf16 away from zero
    val = Fraction(struct.unpack(">f", struct.pack(">I", bits))[0])

    def v(h):
        if (h & 0x7F80) == 0x7F80:  # overflowed into infinity
            return None
        return Fraction(struct.unpack(">f", struct.pack(">I", (h & 0xFFFF) << 16))[0])

    vl, vh = v(lo), v(hi)
    if vh is None:
        # between max finite and infinity: midpoint at the would-be next value
        top = abs(vl) + (abs(vl) - abs(v(lo - 1)))
        dl, dh = abs(val) - abs(vl), top - abs(val)
    else:
        dl, dh = abs(val - vl), abs(vh - val)
    if dl < dh:
        return lo
    if dh < dl:
        return hi & 0xFFFF
    return lo if (lo & 1) == 0 else hi & 0xFFFF


def test_workload_table():
    w = gi.WORKLOADS
    assert (w["f32_256"].M, w["f32_256"].N, w["f32_256"].K) == (256, 256, 256)
    assert w["f32_4096"].flop == 2 * 4096 ** 3
    r = w["f32_ragged"]
    assert (r.M, r.N, r.K, r.alpha, r.beta, r.dist) == (1000, 1500, 777, 1.5, -0.5, "normal")
    b = w["bf16_8192"]
    assert b.dtype == "bf16" and b.b_col_major and b.K == 8192
    t = w["f32_tall"]
    assert (t.M, t.N, t.K) == (16384, 128, 4096)
    h = w["f16_8192"]
    assert h.dtype == "f16" and h.b_col_major and (h.M, h.N, h.K) == (8192, 8192, 8192)
    e = w["f32_8192"]
    assert e.dtype == "f32" and not e.b_col_major and (e.M, e.N, e.K) == (8192, 8192, 8192)
    f = w["bf16_few"]
    assert f.dtype == "bf16" and f.b_col_major and (f.M, f.N, f.K) == (1024, 1024, 16384)
    assert [x.seed for x in w.values()] == [1001, 1002, 1003, 1004, 1005, 1006, 1007, 1008]


def test_determinism_and_layout():
    a = gi.make_inputs(33, 17, 9, dist="normal", beta=1.0, seed=5)
    b = gi.make_inputs(33, 17, 9, dist="normal", beta=1.0, seed=5)
    c = gi.make_inputs(33, 17, 9, dist="normal", beta=1.0, seed=6)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B) and np.array_equal(a.C, b.C)
    assert not np.array_equal(a.A, c.A)
    assert a.A.shape == (33, 9) and a.B.shape == (9, 17) and a.C.shape == (33, 17)
    assert (a.lda, a.ldb, a.ldc) == (9, 17, 17)
    h = gi.make_inputs(33, 17, 9, dtype="bf16", seed=5)
    assert h.B.shape == (17, 9) and h.ldb == 9 and h.C is None and h.A.dtype == np.uint16
    # draw order A, B, C in storage order
    rng = np.random.Generator(np.random.PCG64(5))
    a0 = rng.standard_normal(33 * 9, dtype=np.float32)
    assert np.array_equal(a.A.ravel(), a0)
    u = gi.make_inputs(8, 8, 8, dist="uniform", seed=1)
    assert u.A.min() >= -1 and u.A.max() <= 1


def test_bf16_rne_against_exact_rounding():
    rng = np.random.Generator(np.random.PCG64(9))
    x = np.concatenate([
        rng.standard_normal(3000, dtype=np.float32),
        rng.uniform(-1e-38, 1e-38, 300).astype(np.float32),  # subnormal range
        (rng.standard_normal(300) * 1e30).astype(np.float32),
    ])
    # exact ties: low half-word 0x8000 with even and odd kept LSB
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00008000,
                     0x00018000, 0x7F7F8000, 0x7F7E8000, 0x3F80FFFF, 0x3F807FFF],
                    np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    got = gi.f32_to_bf16_bits(x)
    want = np.array([_bf16_rne_exact(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)
    assert gi.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_bf16_rne_matches_torch_cpu_cast():
    rng = np.random.Generator(np.random.PCG64(10))
    x = rng.standard_normal(100000, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gi.f32_to_bf16_bits(x), t)


def test_bf16_widening_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = gi.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(gi.f32_to_bf16_bits(f[finite]), bits[finite])


@pytest.mark.parametrize("v", [-16, -3, 0, 1, 7, 16])
def test_small_integers_are_bf16_exact(v):
    h = gi.f32_to_bf16_bits(np.array([v], np.float32))
    assert gi.bf16_bits_to_f32(h)[0] == v


def test_f16_rne_against_python_half_packing():
    # struct's 'e' format packs an IEEE binary16 with round-half-to-even, independently of numpy
    import struct
    rng = np.random.Generator(np.random.PCG64(12))
    x = np.concatenate([rng.standard_normal(3000, dtype=np.float32),
                        rng.uniform(-6e-5, 6e-5, 300).astype(np.float32),  # fp16 subnormal range
                        rng.uniform(-65000, 65000, 300).astype(np.float32),
                        # exact ties between neighbouring fp16 values (1 + 2^-11, 1 + 3*2^-11)
                        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -11), 2 ** -25,
                                  3 * 2 ** -25, 0.0, -0.0], np.float32)])
    got = gi.f32_to_f16_bits(x)
    want = np.array([struct.unpack("<H", struct.pack("<e", float(v)))[0] for v in x], np.uint16)
    assert np.array_equal(got, want)
    assert gi.f32_to_f16_bits(np.array([70000.0, -1e9], np.float32)).tolist() == [0x7C00, 0xFC00]

