"""Measured instruction counts of every ladder rung against the closed forms of the pages'
accounting (CPU only: the counts come from the committed rocprofv3 --pmc record).

"【infra之路】理解 Register Tiling", opening section: with one output per thread and 32-wide
tiles, each output element costs 64 shared-memory reads per tile pass (32 of A, 32 of B). Its
key-loop section and three-version comparison: a thread that owns a TM x TN micro-tile reads TM
values of A and TN of B per k and does TM * TN FMAs, so shared reads per FMA fall to
(TM + TN) / (TM * TN), 0.5 for 4 x 4. The counts below are that accounting per wave and per
instruction, for the instruction forms the gfx950 build uses: 16-byte `ds_read_b128` fragment
reads (4 floats, or 8 bf16 of one MFMA fragment), `ds_read2_b32` pairs in the LDS rung,
`ds_write2_b32` pairs for the transposed A stores and `ds_write_b128` for B stores. Any change
of tiling, staging or a stray extra LDS access shows up as a mismatch.

`profiles/lds_counters_ladder_f32_4096_bf16_8192.json` holds the means per dispatch from the
ladder run (fp32 rungs at 4096^3, 16-bit rungs at 8192^3).
"""
from __future__ import annotations

import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD = os.path.join(ROOT, "profiles", "lds_counters_ladder_f32_4096_bf16_8192.json")
K = {"f32_4096": 4096, "bf16_8192": 8192}


@pytest.fixture(scope="module")
def kernels():
    with open(RECORD) as f:
        return json.load(f)["kernels"]


def _find(kernels, prefix):
    hits = [v for k, v in kernels.items() if k.startswith(prefix)]
    assert len(hits) == 1, (prefix, list(kernels))
    return hits[0]


def regtile_lds_per_wave(k, bm, bn, bk, tm, tn, threads=256):
    """Square / small-tile kernels: per slab of bk, tm/4 + tn/4 fragment reads per k; staging of
    the A tile (bm x bk floats, float4 chunks per thread written as 4 scalars down a k-major
    column, two per ds_write2_b32) and the B tile (bk x bn floats, one ds_write_b128 per chunk)."""
    reads = (tm // 4 + tn // 4) * bk
    a_chunks = bm * bk // (4 * threads)
    b_chunks = bk * bn // (4 * threads)
    return (k // bk) * (reads + 2 * a_chunks + b_chunks)


def test_lds_rung_reads_64_values_per_output_per_tile_pass(kernels):
    # 32 x 32 tile, one output per thread: per 32-deep pass 32 values of A and 32 of B (the
    # page's 64), paired into 32 ds_read2_b32, plus one store of A and one of B
    r = _find(kernels, "f32_lds_kernel")
    assert r["lds_instructions_per_wave"] == (K["f32_4096"] // 32) * (64 // 2 + 2)


def test_square_8x16_micro_tile(kernels):
    # 128 x 256 tile, BK 16, 8 x 16 micro-tile: 6 reads per k for 128 FMAs (0.19 floats per FMA)
    r = _find(kernels, "f32_regtile_kernel<SquareCfg")
    assert r["lds_instructions_per_wave"] == regtile_lds_per_wave(K["f32_4096"], 128, 256, 16, 8, 16)
    fma = 8 * 16 * K["f32_4096"]
    assert fma <= r["valu_instructions_per_wave"] <= 1.03 * fma  # FMAs plus a few % of overhead


def test_small_4x4_micro_tile(kernels):
    # 64 x 64 tile, BK 32, 4 x 4 micro-tile: 2 reads per k for 16 FMAs (the page's 0.5 floats
    # per FMA, 4x fewer than one output per thread)
    r = _find(kernels, "f32_regtile_kernel<SmallCfg")
    assert r["lds_instructions_per_wave"] == regtile_lds_per_wave(K["f32_4096"], 64, 64, 32, 4, 4)
    fma = 4 * 4 * K["f32_4096"]
    assert fma <= r["valu_instructions_per_wave"] <= 1.05 * fma


def test_split_k_8_waves(kernels):
    # 64 x 128 tile, 8 waves each over K/8 with its own slabs (BK 8, 64 lanes stage 64 x 8 of A
    # and 8 x 128 of B), then the fixed-order reduction of the 64 x 128 partials (32 float4
    # per lane each): waves 4-7 write, waves 0-3 read; waves 0-3 write, all 8 waves read their
    # eighth of the four partials (16 float4 per lane)
    r = _find(kernels, "f32_splitk_kernel<SplitCfg<8, 8, 16, 8,")
    k_wave = K["f32_4096"] // 8
    per_slab = (8 // 4 + 16 // 4) * 8 + 2 * (64 * 8 // (4 * 64)) + 8 * 128 // (4 * 64)
    reduction = (4 * 32 + 4 * 32 + 4 * 32 + 8 * 16) / 8
    assert r["lds_instructions_per_wave"] == (k_wave // 8) * per_slab + reduction
    fma = 8 * 16 * k_wave
    assert fma <= r["valu_instructions_per_wave"] <= 1.06 * fma


@pytest.mark.parametrize("mf,ksteps_per_slab", [(32, 4), (16, 2)])
def test_mfma_fragment_reads_and_instructions(kernels, mf, ksteps_per_slab):
    # 256 x 256 tile, 2 x 2 waves of 128 x 128, 64-deep slabs: per k step one 16-byte read per
    # A and per B fragment (128 / mf each) and (128 / mf)^2 MFMAs; the first k step's fragments
    # are read once more before the loop
    r = _find(kernels, f"bf16_mfma_dma_kernel<256, 256, 64, 2, 2, {mf},")
    kk = K["bf16_8192"]
    frags = 128 // mf
    reads_per_step = 2 * frags
    assert r["lds_instructions_per_wave"] == reads_per_step + (kk // 64) * ksteps_per_slab * reads_per_step
    assert r["mfma_instructions_per_wave"] == frags * frags * (kk // (64 // ksteps_per_slab))
    assert r["lds_bank_conflict_cycles"] == 0  # the slab swizzle keys


def test_values_read_per_fma_follow_the_pages_accounting(kernels):
    # LDS values read per FMA from the measured counts (store instructions taken out): 2 for one
    # output per thread (2 values per ds_read2_b32), (4 + 4) / 16 = 0.5 for 4 x 4 -- the page's
    # "4x fewer" -- and (8 + 16) / 128 = 0.1875 for 8 x 16 (4 values per ds_read_b128)
    k = K["f32_4096"]
    lds = _find(kernels, "f32_lds_kernel")["lds_instructions_per_wave"]
    assert (lds - 2 * (k // 32)) * 2 / k == 2.0
    small = _find(kernels, "f32_regtile_kernel<SmallCfg")["lds_instructions_per_wave"]
    assert (small - 6 * (k // 32)) * 4 / (16 * k) == 0.5
    square = _find(kernels, "f32_regtile_kernel<SquareCfg")["lds_instructions_per_wave"]
    assert (square - 8 * (k // 16)) * 4 / (128 * k) == 0.1875
