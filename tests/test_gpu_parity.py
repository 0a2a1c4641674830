"""GPU parity of the HIP library against the fp64 CPU oracle, through the C ABI.

Bar: every compared element satisfies |C_gpu - C_ref| <= 1e-5 * (|alpha| sum_k |a_ik b_kj|
+ |beta c_ij|) (oracle.check), and integer-valued inputs, whose every partial sum is exact
in fp32, must match bitwise. Small and ragged problems are compared in full; the full-size
workloads run in the launch configuration the benchmark times and are compared in full too;
larger or rarer cases use a stratified sample (a whole leading tile, the whole last tile row
and column, 65536 seeded positions) that the oracle computes entry by entry.
"""
from __future__ import annotations

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import register_tiled_matrix_amd as rt
from gpu_util import (announce, assert_parity_full, assert_parity_sampled, device_operands, run,
                      sample_positions, workload_reference)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

F32_ALGOS = [rt.ALGO_F32_NAIVE, rt.ALGO_F32_LDS, rt.ALGO_F32_REGTILE, rt.ALGO_F32_SPLITK,
             rt.ALGO_F32_REGTILE_SMALL, rt.ALGO_F32_AUTO]
BF16_ALGOS = [rt.ALGO_BF16_NAIVE, rt.ALGO_BF16_MFMA, rt.ALGO_BF16_MFMA_16X16, rt.ALGO_BF16_AUTO]
BF16_MFMA_ALGOS = [rt.ALGO_BF16_MFMA, rt.ALGO_BF16_MFMA_16X16]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.load()
    yield


# ---- the five workloads ----------------------------------------------------------------
@pytest.mark.parametrize("algo", F32_ALGOS)
def test_f32_256_full(algo):
    inp = gi.workload_inputs(gi.WORKLOADS["f32_256"])
    announce(f"f32_256 algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    assert_parity_full(inp, got, f"f32_256 algo {algo} ({rt.last_kernel()})")


@pytest.mark.parametrize("algo", F32_ALGOS)
def test_f32_ragged_full(algo):
    inp = gi.workload_inputs(gi.WORKLOADS["f32_ragged"])
    announce(f"f32_ragged algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    assert_parity_full(inp, got, f"f32_ragged algo {algo} ({rt.last_kernel()})")


# The full-size workloads through the entry point and launch configuration the benchmark
# times, compared with the oracle over all of C. The exact kernel is asserted, so a change of
# the default dispatch cannot leave the timed kernel untested. Cases of one workload are
# adjacent, so its oracle is computed once.
BENCH_KERNELS = [
    ("f32_4096", rt.ALGO_F32_AUTO, "f32_regtile_128x256x16_8x16_va_vb_vc"),
    ("f32_tall", rt.ALGO_F32_AUTO, "f32_regtile_splitk8_64x128x8_8x16"),
    ("f32_8192", rt.ALGO_F32_AUTO, "f32_regtile_128x256x16_8x16_va_vb_vc"),
    ("bf16_8192", rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_256x256x64_w2x2"),
    ("bf16_8192", rt.ALGO_BF16_MFMA_16X16, "bf16_mfma16x16x32_dma_256x256x64_w2x2"),
    ("f16_8192", rt.ALGO_BF16_AUTO, "f16_mfma32x32x16_dma_256x256x64_w2x2"),
    ("f16_8192", rt.ALGO_BF16_MFMA_16X16, "f16_mfma16x16x32_dma_256x256x64_w2x2"),
]


@pytest.mark.parametrize("wname,algo,kernel", BENCH_KERNELS, ids=[f"{w}-{a}" for w, a, _ in BENCH_KERNELS])
def test_workload_full(wname, algo, kernel):
    inp, ref, mag = workload_reference(wname)
    announce(f"{wname} algo={algo} full comparison")
    got = run(inp, torch, algo).cpu().numpy()
    assert rt.last_kernel() == kernel, rt.last_kernel()
    ok, worst = oracle.check(got, ref, mag)
    assert ok, f"{wname} ({kernel}): worst |err|/bound = {worst:.3g} over all {got.size} entries"


# The benchmarked kernels' resources as the HIP runtime reports them: no spills, and the
# occupancy each design states (two waves per SIMD for the fp32 kernels, whose FMA issue needs
# two; one for the bf16 kernel, whose 256 accumulators per lane fill the AGPRs).
BENCH_RESOURCES = [("f32_4096", 256, 2), ("f32_tall", 512, 2), ("f32_ragged", 512, 2), ("bf16_8192", 256, 1)]


@pytest.mark.parametrize("wname,threads,waves", BENCH_RESOURCES, ids=[w for w, _, _ in BENCH_RESOURCES])
def test_benchmarked_kernels_resources(wname, threads, waves):
    w = gi.WORKLOADS[wname]
    inp = gi.make_inputs(w.M, w.N, w.K, dtype=w.dtype, dist="normal", alpha=w.alpha, beta=w.beta, seed=1)
    announce(f"{wname} kernel resources")
    run(inp, torch)
    info = rt.last_kernel_info()
    assert info["scratch_bytes"] == 0, info
    assert info["workgroup_size"] == threads, info
    assert info["waves_per_simd"] == waves, info
    assert info["registers"] <= 512 // waves, info


def test_f32_ragged_default_kernel():
    inp = gi.workload_inputs(gi.WORKLOADS["f32_ragged"])
    announce("f32_ragged default entry point")
    got = run(inp, torch).cpu().numpy()
    # 1000 x 1500 is 256 tiles of 64x96 (one per CU) against 192 of 64x128
    assert rt.last_kernel() == "f32_regtile_splitk8_64x96x8_8x12_guard", rt.last_kernel()
    assert_parity_full(inp, got, "f32_ragged default")


def _integer_inputs(wname, seed):
    """A workload's shape and layout with integer entries in [-16, 16]: every product and
    partial sum is an integer below 2^24 in magnitude (K <= 8192), so any summation order is
    exact in fp32 and the result must equal the oracle bitwise."""
    w = gi.WORKLOADS[wname]
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.integers(-16, 17, (w.M, w.K)).astype(np.float32)
    if w.dtype == "f32":
        return gi.GemmInputs(w.M, w.N, w.K, 1.0, 0.0, "f32", False, A, rng.integers(-16, 17, (w.K, w.N)).astype(np.float32), None)
    to_bits = gi.f32_to_bf16_bits if w.dtype == "bf16" else gi.f32_to_f16_bits
    Bt = rng.integers(-16, 17, (w.N, w.K)).astype(np.float32)
    return gi.GemmInputs(w.M, w.N, w.K, 1.0, 0.0, w.dtype, True, to_bits(A.ravel()).reshape(w.M, w.K),
                         to_bits(Bt.ravel()).reshape(w.N, w.K), None)


@pytest.mark.parametrize("wname,kernel", [("f32_4096", "f32_regtile_128x256x16_8x16_va_vb_vc"),
                                          ("bf16_8192", "bf16_mfma32x32x16_dma_256x256x64_w2x2")])
def test_workload_integer_inputs_bitwise_full(wname, kernel):
    inp = _integer_inputs(wname, 4242)
    announce(f"{wname} integer inputs, full bitwise comparison")
    got = run(inp, torch).cpu().numpy()
    assert rt.last_kernel() == kernel, rt.last_kernel()
    ref, _ = oracle.gemm_inputs(inp)
    assert np.array_equal(got.astype(np.float64), ref)


# ---- bf16 at a size the oracle finishes in full -----------------------------------------
@pytest.mark.parametrize("algo", BF16_ALGOS)
@pytest.mark.parametrize("shape", [(512, 768, 1024), (300, 257, 777), (1024, 1024, 256),
                                   (2048, 4096, 192)])
def test_bf16_full(algo, shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="bf16", dist="normal", alpha=1.5, beta=-0.5, seed=M + N + K)
    announce(f"bf16 {shape} algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    if shape == (2048, 4096, 192) and algo != rt.ALGO_BF16_NAIVE:
        assert "_dma_" in rt.last_kernel()  # full aligned 256x256 tiles take the LDS-DMA kernel
    assert_parity_full(inp, got, f"bf16 {shape} algo {algo} ({rt.last_kernel()})")


# ---- edges: every tile boundary on either side ---------------------------------------------
EDGE_SHAPES = [(1, 1, 1), (1, 7, 3), (2, 3, 5), (3, 1, 2), (17, 33, 9), (127, 129, 15),
               (128, 128, 16), (129, 127, 17), (255, 257, 63), (256, 256, 64), (257, 255, 65),
               (131, 293, 300), (64, 1024, 31), (1000, 8, 100), (8, 1000, 1000)]


@pytest.mark.parametrize("algo", [rt.ALGO_F32_REGTILE, rt.ALGO_F32_SPLITK, rt.ALGO_F32_REGTILE_SMALL])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in EDGE_SHAPES])
def test_f32_regtile_edges(shape, algo):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=-1.25, beta=0.75, seed=M * 7 + N + K)
    announce(f"f32 edges {shape} algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    assert_parity_full(inp, got, f"f32 edges {shape} ({rt.last_kernel()})")


# Split-K shapes with at least 192 tiles of 64x128, which take an 8-wave kernel: 64x128 tiles
# of 8x16 micro-tiles, or 64x96 tiles of 8x12 where those need fewer rounds of 256 workgroups
# times tile area. Ragged M, N and K; K below the 8 waves x 8 of one slab each (waves past K
# add zeros); N below one tile; exact multiples (no bounds checks).
SPLITK8_SHAPES = [(13000, 50, 37, 96), (12289, 130, 1283, 96), (8192, 256, 1300, 128),
                  (12800, 128, 1536, 128), (12352, 1, 7, 96), (16384, 96, 2048, 96), (1000, 1500, 777, 96),
                  (12288, 192, 2048, 96)]


@pytest.mark.parametrize("shape", SPLITK8_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k, _ in SPLITK8_SHAPES])
def test_f32_splitk8_edges(shape):
    M, N, K, tile_n = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=-1.25, beta=0.75, seed=M + N + K)
    announce(f"f32 split-K 8 waves {shape}")
    got = run(inp, torch, rt.ALGO_F32_SPLITK).cpu().numpy()
    name = rt.last_kernel()
    micro = {128: "8x16", 96: "8x12"}[tile_n]
    assert name.startswith(f"f32_regtile_splitk8_64x{tile_n}x8_{micro}"), name
    assert name.endswith("_guard") == (M % 64 != 0 or N % tile_n != 0 or K % 64 != 0), name
    assert_parity_full(inp, got, f"f32 split-K {shape} ({name})")


# Split-K on 32x32 tiles (8 waves, 4x4 micro-tiles), taken for fewer than 64 tiles of 64x64:
# exact multiples of the tile and of BK 16 (no bounds checks), ragged M, N and K, K below one
# slab per wave, one row or column, and a long K.
SPLITK_TINY_SHAPES = [(256, 256, 256), (64, 96, 1024), (255, 257, 255), (1, 500, 300), (500, 1, 300),
                      (33, 31, 17), (32, 32, 16), (200, 300, 64), (100, 100, 10000), (448, 480, 97)]


# Split-K with eight waves on each 64x64 tile (8x8 micro-tiles), taken for 64 to 447 tiles of
# 64x64 when fewer than 192 tiles of 64x128 exist: whole tiles and slabs, ragged M, N and K, a
# K below eight slabs, and a long K.
SPLITK8_64_SHAPES = [(1024, 1024, 1024), (512, 512, 4096), (1000, 1000, 3000), (900, 700, 1500),
                     (1024, 768, 100), (513, 511, 257), (768, 768, 8192)]


@pytest.mark.parametrize("shape", SPLITK8_64_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SPLITK8_64_SHAPES])
def test_f32_splitk8_64x64_tiles(shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=1.5, beta=-0.5, seed=M + 5 * N + K)
    announce(f"f32 split-K 8 waves 64x64 {shape}")
    got = run(inp, torch, rt.ALGO_F32_SPLITK).cpu().numpy()
    name = rt.last_kernel()
    assert name.startswith("f32_regtile_splitk8_64x64x16_8x8"), name
    assert name.endswith("_guard") == (M % 64 != 0 or N % 64 != 0 or K % 16 != 0), name
    assert_parity_full(inp, got, f"f32 split-K 8 waves 64x64 {shape} ({name})")


# Split-K with four waves on each 64x64 tile (8x8 micro-tiles): 448 or more such tiles (two
# workgroups per CU) with K below 1280. Whole tiles and slabs, and ragged M, N and K.
SPLITK4_64_SHAPES = [(2048, 1024, 1024), (1500, 1300, 700), (1409, 1313, 129)]


@pytest.mark.parametrize("shape", SPLITK4_64_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SPLITK4_64_SHAPES])
def test_f32_splitk4_64x64_tiles(shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=-0.75, beta=1.25, seed=M + 7 * N + K)
    announce(f"f32 split-K 4 waves 64x64 {shape}")
    got = run(inp, torch, rt.ALGO_F32_SPLITK).cpu().numpy()
    name = rt.last_kernel()
    assert name.startswith("f32_regtile_splitk4_64x64x16_8x8"), name
    assert name.endswith("_guard") == (M % 64 != 0 or N % 64 != 0 or K % 16 != 0), name
    assert_parity_full(inp, got, f"f32 split-K 4 waves 64x64 {shape} ({name})")


@pytest.mark.parametrize("shape", SPLITK_TINY_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SPLITK_TINY_SHAPES])
def test_f32_splitk_32x32_tiles(shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=1.5, beta=-0.5, seed=M + 3 * N + K)
    announce(f"f32 split-K 32x32 {shape}")
    got = run(inp, torch, rt.ALGO_F32_SPLITK).cpu().numpy()
    name = rt.last_kernel()
    assert name.startswith("f32_regtile_splitk8_32x32x16_4x4"), name
    assert name.endswith("_guard") == (M % 32 != 0 or N % 32 != 0 or K % 16 != 0), name
    assert_parity_full(inp, got, f"f32 split-K 32x32 {shape} ({name})")


def test_f32_auto_picks_by_tile_count():
    # square kernel from 384 tiles of 128x256; split-K below that for a long enough K (eight
    # waves per 64x64 tile below 448 of them from K >= 128, 32x32 tiles below 64 of them from
    # K >= 64); otherwise the small-tile kernel
    cases = [((4096, 3072, 64), "f32_regtile_128x256x16_8x16"), ((4096, 2048, 2048), "f32_regtile_splitk8"),
             ((4096, 2048, 1024), "f32_regtile_splitk4"),
             ((1000, 1500, 777), "f32_regtile_splitk8"), ((1024, 1024, 1024), "f32_regtile_splitk8_64x64x16_8x8"),
             ((3000, 2000, 512), "f32_regtile_64x64x32_4x4"), ((1000, 1500, 300), "f32_regtile_splitk8_64x96"),
             ((1000, 1500, 100), "f32_regtile_64x64x32_4x4"), ((1024, 1024, 128), "f32_regtile_splitk8_64x64"),
             ((1280, 1792, 256), "f32_regtile_64x64x32_4x4"),
             ((256, 256, 256), "f32_regtile_splitk8_32x32x16_4x4"), ((500, 400, 64), "f32_regtile_splitk8_32x32"),
             ((256, 256, 48), "f32_regtile_64x64x32_4x4"), ((512, 512, 63), "f32_regtile_64x64x32_4x4"),
             ((512, 512, 256), "f32_regtile_splitk8_64x64x16_8x8")]
    for (M, N, K), prefix in cases:
        A = torch.zeros((M, K), device="cuda")
        B = torch.zeros((K, N), device="cuda")
        rt.gemm_f32(A, B)
        assert rt.last_kernel().startswith(prefix), ((M, N, K), rt.last_kernel())
        At = torch.zeros((K, M), device="cuda").t()
        rt.gemm_f32(At, B)  # transposed A: split-K stages row-major operands only
        assert "splitk" not in rt.last_kernel(), ((M, N, K), rt.last_kernel())
    torch.cuda.synchronize()


@pytest.mark.parametrize("algo", BF16_MFMA_ALGOS)
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in EDGE_SHAPES])
def test_bf16_mfma_edges(shape, algo):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="bf16", dist="normal", alpha=-1.25, beta=0.75, seed=M * 7 + N + K)
    announce(f"bf16 edges {shape} algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    assert_parity_full(inp, got, f"bf16 edges {shape}")


# ---- LDS-DMA kernel on tiles cut by M or N ---------------------------------------------------
# At least 128 tiles of 256x256 counting partial ones, K a whole number of 64-deep slabs: the
# DMA kernel, whose descriptors stop at the last real row of A, B and C. C has padded rows, and
# the padding (columns N.. of every row) must stay untouched.
DMA_RAGGED = [("bf16", (8000, 4100, 128), 1.5, -0.5, "full"), ("bf16", (4097, 8191, 64), 1.0, 0.0, "full"),
              ("f16", (4100, 8000, 192), -1.0, 0.5, "full"), ("bf16", (2049, 4095, 3072), 1.0, 0.0, "sampled")]


@pytest.mark.parametrize("dtype,shape,alpha,beta,mode", DMA_RAGGED,
                         ids=[f"{d}-{'x'.join(map(str, s))}" for d, s, _, _, _ in DMA_RAGGED])
def test_16bit_dma_kernel_on_ragged_m_n(dtype, shape, alpha, beta, mode):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=alpha, beta=beta, seed=M + 2 * N + K)
    announce(f"{dtype} DMA ragged {shape}")
    A, B, C0 = device_operands(inp, torch)
    big = torch.full((M, N + 7), 1234.5, device="cuda")
    C = big[:, :N]
    if inp.C is not None:
        C.copy_(C0)
    fn = {"bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, B, C, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    name = rt.last_kernel()
    assert "_dma_" in name, name
    assert torch.all(big[:, N:] == 1234.5).item(), "a store landed past column N"
    got = C.cpu().numpy()
    if mode == "full":
        assert_parity_full(inp, got, f"{dtype} {shape} ({name})")
    else:
        assert_parity_sampled(inp, got, f"{dtype} {shape} ({name})")


# K ending inside the last 64-deep slab (K a multiple of 8): that slab's chunks past K load as
# zeros on both operands.
DMA_KTAIL = [("bf16", rt.ALGO_BF16_MFMA, (4096, 4096, 1000)), ("bf16", rt.ALGO_BF16_MFMA, (4100, 8000, 8)),
             ("f16", rt.ALGO_BF16_MFMA, (8192, 4096, 72)), ("bf16", rt.ALGO_BF16_MFMA_16X16, (4096, 4096, 1000)),
             ("bf16", rt.ALGO_BF16_MFMA, (3999, 4101, 1000))]


@pytest.mark.parametrize("dtype,algo,shape", DMA_KTAIL,
                         ids=[f"{d}-{a}-{'x'.join(map(str, s))}" for d, a, s in DMA_KTAIL])
def test_16bit_dma_kernel_k_tail(dtype, algo, shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=-0.5, seed=M + N + 3 * K)
    announce(f"{dtype} DMA K tail algo={algo} {shape}")
    got = run(inp, torch, algo).cpu().numpy()
    name = rt.last_kernel()
    assert "_dma_" in name and name.endswith("_ktail"), name
    if M * N * K <= 5_000_000_000:
        assert_parity_full(inp, got, f"{dtype} {shape} ({name})")
    else:
        assert_parity_sampled(inp, got, f"{dtype} {shape} ({name})")


def test_16bit_dma_kernel_k_tail_integer_bitwise():
    # any value read past K (garbage beyond the row's end) would show in an exact result
    rng = np.random.Generator(np.random.PCG64(81))
    M, N, K = 4096, 4096, 1000
    A = gi.f32_to_bf16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_bf16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, A, Bt, None)
    announce("bf16 DMA K tail integer bitwise")
    got = run(inp, torch).cpu().numpy()
    assert rt.last_kernel().endswith("_ktail"), rt.last_kernel()
    I, J = sample_positions(M, N, seed=3)
    ref, _ = oracle.gemm_inputs_entries(inp, I, J)
    assert np.array_equal(got[I, J].astype(np.float64), ref)


# ---- 16-bit split-K kernel: 64x64 tiles, K dealt out to the 4 waves of a workgroup ------------
# Full comparisons on shapes with ragged tile edges, K tails (K a multiple of 8 ending inside a
# 64-deep slab, or inside the first 16-wide block), fewer slabs than waves, and C with padded
# rows (ldc = N + 5: scalar stores) whose padding must stay untouched.
SK16_SHAPES = [(1024, 1024, 4096), (1000, 1000, 776), (64, 64, 64), (1, 2, 8), (65, 129, 72),
               (300, 257, 1000), (2048, 512, 8192), (128, 64, 200), (64, 64, 16), (100, 100, 8)]


@pytest.mark.parametrize("pad", [0, 5])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SK16_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SK16_SHAPES])
def test_16bit_splitk_kernel(shape, dtype, pad):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.5, beta=-0.5, seed=M + 3 * N + K + pad)
    announce(f"{dtype} split-K {shape} pad {pad}")
    A, B, C0 = device_operands(inp, torch)
    big = torch.full((M, N + pad), 1234.5, device="cuda")
    C = big[:, :N]
    C.copy_(C0)
    fn = {"bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, B, C, alpha=inp.alpha, beta=inp.beta, algo=rt.ALGO_BF16_MFMA_SPLITK)
    torch.cuda.synchronize()
    name = rt.last_kernel()
    assert name == f"{dtype}_mfma32x32x16_splitk4_64x64x64" + ("_ktail" if K % 64 else ""), name
    if pad:
        assert torch.all(big[:, N:] == 1234.5).item(), "a store landed past column N"
    assert_parity_full(inp, C.cpu().numpy(), f"{dtype} split-K {shape} pad {pad}")


def test_16bit_auto_picks_splitk_by_tile_count():
    # the default entry points: split-K for few 64x64 tiles with enough K, the LDS-DMA kernel
    # otherwise
    cases = [((1024, 1024, 4096), "splitk4"), ((512, 512, 1024), "splitk4"), ((1280, 1280, 8192), "splitk4"),
             ((1024, 1024, 512), "_dma_"), ((1024, 2048, 2048), "_dma_"), ((1536, 1536, 8192), "_dma_")]
    for (M, N, K), want in cases:
        A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        Bt = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
        rt.gemm_bf16(A, Bt.t())
        assert want in rt.last_kernel(), ((M, N, K), rt.last_kernel())
        rt.gemm_f16(A.half(), Bt.half().t())
        assert want in rt.last_kernel() and rt.last_kernel().startswith("f16_"), ((M, N, K), rt.last_kernel())
    # other storage orders: up to 256 tiles with K >= 1024 in all of them; up to 512 with K >=
    # 4096 only for "t n" (and "n t" above)
    def storage(M, N, K, ta, tb):
        A = torch.zeros((K, M) if ta else (M, K), dtype=torch.bfloat16, device="cuda")
        B = torch.zeros((N, K) if tb else (K, N), dtype=torch.bfloat16, device="cuda")
        return (A.t() if ta else A), (B.t() if tb else B)
    for (M, N, K), (ta, tb), want in (((1024, 1024, 4096), (0, 0), "splitk4_64x64x64_nn"),
                                      ((1024, 1024, 4096), (1, 1), "splitk4_64x64x64_tt"),
                                      ((1024, 1024, 4096), (1, 0), "splitk4_64x64x64_tn"),
                                      ((1024, 2048, 8192), (1, 0), "splitk4_64x64x64_tn"),
                                      ((1024, 2048, 8192), (0, 0), "_dma_"),
                                      ((1024, 2048, 8192), (1, 1), "_dma_")):
        A, B = storage(M, N, K, ta, tb)
        rt.gemm_bf16(A, B)
        assert want in rt.last_kernel(), ((M, N, K), (ta, tb), rt.last_kernel())
    torch.cuda.synchronize()


def test_16bit_splitk_integer_inputs_bitwise():
    # |partial sums| <= 4104 * 256, exact in fp32: the sum over the four waves' partials must
    # equal the oracle bit for bit (K tail included)
    rng = np.random.Generator(np.random.PCG64(81))
    M, N, K = 1000, 1000, 4104
    A = gi.f32_to_bf16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_bf16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, A, Bt, None)
    announce("bf16 split-K integer bitwise")
    got = run(inp, torch, rt.ALGO_BF16_MFMA_SPLITK).cpu().numpy()
    assert rt.last_kernel() == "bf16_mfma32x32x16_splitk4_64x64x64_ktail", rt.last_kernel()
    ref, _ = oracle.gemm_inputs(inp)
    assert np.array_equal(got.astype(np.float64), ref)


def test_16bit_splitk_falls_back_where_it_does_not_apply():
    # K not a multiple of 8 with a K-contiguous operand, and an M-contiguous A whose column count
    # and leading dimension are not multiples of 8: the split-K rung hands the problem to the
    # MFMA kernel, with the same results as that rung
    for (M, N, K), ta in (((300, 200, 100), False), ((300, 256, 512), True)):
        inp = gi.make_inputs(M, N, K, dtype="bf16", dist="normal", alpha=1.0, beta=0.0, seed=M + N + K)
        A, B, _ = device_operands(inp, torch)
        if ta:
            A = A.t().contiguous().t()
        announce(f"bf16 split-K fallback {(M, N, K)} ta={ta}")
        C1 = rt.gemm_bf16(A, B, algo=rt.ALGO_BF16_MFMA_SPLITK)
        name = rt.last_kernel()
        C2 = rt.gemm_bf16(A, B, algo=rt.ALGO_BF16_MFMA)
        torch.cuda.synchronize()
        assert "splitk" not in name, name
        assert name == rt.last_kernel(), (name, rt.last_kernel())
        assert torch.equal(C1, C2)
        assert_parity_full(inp, C1.cpu().numpy(), f"split-K fallback {(M, N, K)}")


# ---- bitwise: integer-valued operands (every partial sum exact in fp32) ---------------------
@pytest.mark.parametrize("algo", F32_ALGOS)
def test_f32_integer_inputs_are_bitwise_exact(algo):
    rng = np.random.Generator(np.random.PCG64(77))
    M, N, K = 384, 260, 4096
    A = rng.integers(-16, 17, (M, K)).astype(np.float32)
    B = rng.integers(-16, 17, (K, N)).astype(np.float32)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "f32", False, A, B, None)
    announce(f"f32 integer bitwise algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    ref, _ = oracle.gemm_inputs(inp)
    assert np.array_equal(got.astype(np.float64), ref)


def test_bf16_integer_inputs_are_bitwise_exact():
    rng = np.random.Generator(np.random.PCG64(78))
    M, N, K = 256, 512, 8192
    A = gi.f32_to_bf16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_bf16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, A, Bt, None)
    announce("bf16 integer bitwise")
    got = run(inp, torch, rt.ALGO_BF16_MFMA).cpu().numpy()
    ref, _ = oracle.gemm_inputs(inp)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("algo", BF16_MFMA_ALGOS)
def test_bf16_full_tile_integer_inputs_are_bitwise_exact(algo):
    # 128 full 256x256 tiles: the LDS-DMA kernels; |partial sums| <= 2^18, exact in fp32
    rng = np.random.Generator(np.random.PCG64(79))
    M, N, K = 2048, 4096, 1024
    A = gi.f32_to_bf16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_bf16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, A, Bt, None)
    announce(f"bf16 full-tile integer bitwise algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    assert "_dma_" in rt.last_kernel()
    I, J = sample_positions(M, N, seed=3)
    ref, _ = oracle.gemm_inputs_entries(inp, I, J)
    assert np.array_equal(got[I, J].astype(np.float64), ref)


def test_closed_forms_on_gpu():
    n = 300
    eye = np.eye(n, dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(79))
    Bm = rng.standard_normal((n, 200), dtype=np.float32)
    announce("closed forms")
    got = run(gi.GemmInputs(n, 200, n, 1.0, 0.0, "f32", False, eye, Bm, None), torch).cpu().numpy()
    assert np.array_equal(got, Bm)  # identity: C == B bitwise
    ones = gi.GemmInputs(130, 70, 1000, 1.0, 0.0, "f32", False, np.ones((130, 1000), np.float32),
                         np.ones((1000, 70), np.float32), None)
    assert np.all(run(ones, torch).cpu().numpy() == 1000.0)
    hones = gi.GemmInputs(130, 70, 1000, 1.0, 0.0, "bf16", True, np.full((130, 1000), 0x3F80, np.uint16),
                          np.full((70, 1000), 0x3F80, np.uint16), None)
    assert np.all(run(hones, torch).cpu().numpy() == 1000.0)


# ---- fp16 operands (the pages' half-precision GEMM) on the same MFMA kernels -----------------
F16_ALGOS = [rt.ALGO_BF16_NAIVE, rt.ALGO_BF16_MFMA, rt.ALGO_BF16_MFMA_16X16, rt.ALGO_BF16_AUTO]


@pytest.mark.parametrize("algo", F16_ALGOS)
@pytest.mark.parametrize("shape", [(512, 768, 1024), (300, 257, 777), (2048, 4096, 192)])
def test_f16_full(algo, shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f16", dist="normal", alpha=1.5, beta=-0.5, seed=M + N + K + 1)
    announce(f"f16 {shape} algo={algo}")
    got = run(inp, torch, algo).cpu().numpy()
    name = rt.last_kernel()
    assert name.startswith("f16_")
    if shape == (2048, 4096, 192) and algo != rt.ALGO_BF16_NAIVE:
        assert "_dma_" in name
    assert_parity_full(inp, got, f"f16 {shape} algo {algo} ({name})")


@pytest.mark.parametrize("shape", [(1, 1, 1), (17, 33, 9), (129, 127, 17), (257, 255, 65), (131, 293, 300)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f16_mfma_edges(shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f16", dist="normal", alpha=-1.25, beta=0.75, seed=M * 5 + N + K)
    announce(f"f16 edges {shape}")
    got = run(inp, torch, rt.ALGO_BF16_MFMA).cpu().numpy()
    assert_parity_full(inp, got, f"f16 edges {shape}")


@pytest.mark.parametrize("M,N,K", [(256, 512, 2048), (2048, 4096, 1024)])
def test_f16_integer_inputs_are_bitwise_exact(M, N, K):
    # integers in [-16, 16] are exact in fp16; every partial sum stays below 2^24
    rng = np.random.Generator(np.random.PCG64(80 + M))
    A = gi.f32_to_f16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_f16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "f16", True, A, Bt, None)
    announce(f"f16 integer bitwise {M}x{N}x{K}")
    got = run(inp, torch, rt.ALGO_BF16_MFMA).cpu().numpy()
    I, J = sample_positions(M, N, seed=4)
    ref, _ = oracle.gemm_inputs_entries(inp, I, J)
    assert np.array_equal(got[I, J].astype(np.float64), ref)


def test_f16_and_bf16_kernels_differ_only_in_the_element_type():
    # the same 16-bit patterns read as fp16 and as bf16 give different products (a kernel that
    # ignored the element type would pass one of the two parity checks only by accident)
    inp16 = gi.make_inputs(256, 256, 512, dtype="f16", dist="normal", seed=31)
    as_bf16 = gi.GemmInputs(256, 256, 512, 1.0, 0.0, "bf16", True, inp16.A, inp16.B, None)
    announce("f16 vs bf16 element type")
    g16 = run(inp16, torch, rt.ALGO_BF16_MFMA).cpu().numpy()
    g_bf = run(as_bf16, torch, rt.ALGO_BF16_MFMA).cpu().numpy()
    assert_parity_full(inp16, g16, "f16 reading")
    assert_parity_full(as_bf16, g_bf, "bf16 reading of the same bits")
    assert not np.allclose(g16, g_bf)


# ---- epilogue conventions -----------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_beta_zero_never_reads_c(dtype):
    inp = gi.make_inputs(200, 300, 64, dtype=dtype, dist="normal", seed=3)
    announce(f"beta=0 NaN C {dtype}")
    got = run(inp, torch, C_init=torch.full((200, 300), float("nan"), device="cuda")).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert_parity_full(inp, got, "beta=0 with NaN C")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(200, 300, 1024), (1000, 1000, 776)], ids=lambda s: "x".join(map(str, s)))
def test_16bit_splitk_beta_zero_never_reads_c(dtype, shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", seed=5)
    announce(f"beta=0 NaN C {dtype} split-K {shape}")
    got = run(inp, torch, rt.ALGO_BF16_MFMA_SPLITK, C_init=torch.full((M, N), float("nan"), device="cuda"))
    assert "splitk4" in rt.last_kernel(), rt.last_kernel()
    got = got.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert_parity_full(inp, got, "split-K beta=0 with NaN C")


F32_EPILOGUE_CASES = [(rt.ALGO_F32_REGTILE, (200, 300, 64), "f32_regtile_128x256"),
                      (rt.ALGO_F32_REGTILE_SMALL, (200, 300, 64), "f32_regtile_64x64x32"),
                      (rt.ALGO_F32_SPLITK, (200, 300, 64), "f32_regtile_splitk8_32x32"),
                      (rt.ALGO_F32_SPLITK, (1024, 768, 100), "f32_regtile_splitk8_64x64"),
                      (rt.ALGO_F32_SPLITK, (1500, 1300, 300), "f32_regtile_splitk4_64x64"),
                      (rt.ALGO_F32_SPLITK, (13000, 50, 37), "f32_regtile_splitk8"),
                      (rt.ALGO_F32_SPLITK, (12800, 128, 512), "f32_regtile_splitk8")]


@pytest.mark.parametrize("algo,shape,prefix", F32_EPILOGUE_CASES,
                         ids=[f"{a}-{'x'.join(map(str, s))}" for a, s, _ in F32_EPILOGUE_CASES])
def test_f32_beta_zero_never_reads_c_every_kernel(algo, shape, prefix):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=0.5, seed=M + N)
    announce(f"beta=0 NaN C algo={algo} {shape}")
    got = run(inp, torch, algo, C_init=torch.full((M, N), float("nan"), device="cuda")).cpu().numpy()
    assert rt.last_kernel().startswith(prefix), rt.last_kernel()
    assert np.all(np.isfinite(got))
    assert_parity_full(inp, got, f"beta=0 with NaN C ({rt.last_kernel()})")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_alpha_zero_and_k_zero_scale_c(dtype):
    M, N = 70, 90
    rng = np.random.Generator(np.random.PCG64(5))
    C0 = rng.standard_normal((M, N), dtype=np.float32)
    announce(f"alpha=0 / K=0 {dtype}")
    inp = gi.make_inputs(M, N, 33, dtype=dtype, seed=4, beta=-2.0, alpha=0.0)
    inp.C = C0
    A, B, C = device_operands(inp, torch)
    A.fill_(float("nan"))
    fn = {"f32": rt.gemm_f32, "bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, B, C, alpha=0.0, beta=-2.0)
    torch.cuda.synchronize()
    assert rt.last_kernel() == "scale_c"
    assert np.array_equal(C.cpu().numpy(), -2.0 * C0)
    # K == 0 with beta == 0 gives zeros (C not read)
    C2 = torch.full((M, N), float("nan"), device="cuda")
    fn(A[:, :0], B[:0, :], C2, alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C2).item() == 0


# ---- strides, misalignment, streams, determinism --------------------------------------------
def test_f32_strided_and_misaligned_views():
    rng = np.random.Generator(np.random.PCG64(6))
    M, N, K = 300, 260, 301
    big_a = torch.from_numpy(rng.standard_normal((M, K + 9), dtype=np.float32)).cuda()
    big_b = torch.from_numpy(rng.standard_normal((K, N + 5), dtype=np.float32)).cuda()
    big_c = torch.zeros((M, N + 3), device="cuda")
    A = big_a[:, 1:K + 1]  # lda = K + 9, pointer offset by one float
    B = big_b[:, 3:N + 3]
    C = big_c[:, 1:N + 1]
    announce("f32 strided/misaligned")
    rt.gemm_f32(A, B, C)
    torch.cuda.synchronize()
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "f32", False, A.cpu().numpy(), B.cpu().numpy(), None)
    assert_parity_full(inp, C.cpu().numpy(), "strided views")
    assert torch.count_nonzero(big_c[:, 0]).item() == 0  # nothing written outside C
    assert torch.count_nonzero(big_c[:, N + 1:]).item() == 0


def test_bf16_strided_and_misaligned_views():
    rng = np.random.Generator(np.random.PCG64(7))
    M, N, K = 260, 300, 200
    ha = gi.f32_to_bf16_bits(rng.standard_normal(M * (K + 5), dtype=np.float32)).reshape(M, K + 5)
    hb = gi.f32_to_bf16_bits(rng.standard_normal(N * (K + 3), dtype=np.float32)).reshape(N, K + 3)
    da = torch.from_numpy(ha.view(np.int16)).cuda().view(torch.bfloat16)
    db = torch.from_numpy(hb.view(np.int16)).cuda().view(torch.bfloat16)
    A = da[:, 1:K + 1]
    B = db[:, 2:K + 2].t()
    announce("bf16 strided/misaligned")
    C = rt.gemm_bf16(A, B)
    torch.cuda.synchronize()
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, np.ascontiguousarray(ha[:, 1:K + 1]),
                        np.ascontiguousarray(hb[:, 2:K + 2]), None)
    assert_parity_full(inp, C.cpu().numpy(), "bf16 strided views")


@pytest.mark.parametrize("pad_a,pad_b,off_a,splitk", [(16, 8, 0, True), (24, 40, 8, True), (5, 3, 1, False)])
def test_16bit_splitk_padded_rows(pad_a, pad_b, off_a, splitk):
    # leading dimensions beyond K: multiples of 8 with 16-byte aligned rows take the split-K
    # kernel; otherwise the split-K rung hands the problem on (same results either way)
    rng = np.random.Generator(np.random.PCG64(9 + pad_a))
    M, N, K = 333, 190, 1096
    ha = gi.f32_to_bf16_bits(rng.standard_normal(M * (K + pad_a), dtype=np.float32)).reshape(M, K + pad_a)
    hb = gi.f32_to_bf16_bits(rng.standard_normal(N * (K + pad_b), dtype=np.float32)).reshape(N, K + pad_b)
    da = torch.from_numpy(ha.view(np.int16)).cuda().view(torch.bfloat16)
    db = torch.from_numpy(hb.view(np.int16)).cuda().view(torch.bfloat16)
    A = da[:, off_a:off_a + K]
    B = db[:, :K].t()
    announce(f"bf16 split-K padded rows lda={K + pad_a} ldb={K + pad_b} offset={off_a}")
    C = rt.gemm_bf16(A, B, algo=rt.ALGO_BF16_MFMA_SPLITK)
    torch.cuda.synchronize()
    assert ("splitk4" in rt.last_kernel()) == splitk, rt.last_kernel()
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, np.ascontiguousarray(ha[:, off_a:off_a + K]),
                        np.ascontiguousarray(hb[:, :K]), None)
    assert_parity_full(inp, C.cpu().numpy(), f"bf16 split-K padded rows ({rt.last_kernel()})")


def test_runs_on_the_callers_stream_and_is_deterministic():
    inp = gi.make_inputs(1024, 1024, 1024, dist="uniform", seed=8)
    A, B, C = device_operands(inp, torch)
    s = torch.cuda.Stream()
    announce("stream + determinism")
    outs = []
    with torch.cuda.stream(s):
        for _ in range(5):
            C.zero_()
            rt.gemm_f32(A, B, C)
            outs.append(C.clone())
    s.synchronize()
    first = outs[0].cpu().numpy()
    for o in outs[1:]:
        assert np.array_equal(o.cpu().numpy(), first)
    assert_parity_full(inp, first, "stream run")


def test_f32_ladder_rungs_agree_bitwise():
    # the SIMT rungs except split-K accumulate every output with fmaf over k in natural order
    inp = gi.make_inputs(333, 517, 1029, dist="normal", seed=9)
    announce("ladder bitwise agreement")
    outs = [run(inp, torch, a).cpu().numpy() for a in (rt.ALGO_F32_NAIVE, rt.ALGO_F32_LDS,
                                                        rt.ALGO_F32_REGTILE, rt.ALGO_F32_REGTILE_SMALL)]
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


def test_f32_strided_views_every_register_tiled_kernel():
    # unaligned lda/ldb/ldc and pointers offset by one float take the scalar load paths
    rng = np.random.Generator(np.random.PCG64(10))
    M, N, K = 300, 260, 301
    big_a = torch.from_numpy(rng.standard_normal((M, K + 9), dtype=np.float32)).cuda()
    big_b = torch.from_numpy(rng.standard_normal((K, N + 5), dtype=np.float32)).cuda()
    A, B = big_a[:, 1:K + 1], big_b[:, 3:N + 3]
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "f32", False, A.cpu().numpy(), B.cpu().numpy(), None)
    for algo in (rt.ALGO_F32_REGTILE, rt.ALGO_F32_SPLITK, rt.ALGO_F32_REGTILE_SMALL):
        announce(f"f32 strided algo={algo}")
        big_c = torch.zeros((M, N + 3), device="cuda")
        C = big_c[:, 1:N + 1]
        rt.gemm_f32(A, B, C, algo=algo)
        torch.cuda.synchronize()
        name = rt.last_kernel()
        assert "_va" not in name and "_vb" not in name
        assert_parity_full(inp, C.cpu().numpy(), f"strided views ({name})")
        assert torch.count_nonzero(big_c[:, 0]).item() == 0
        assert torch.count_nonzero(big_c[:, N + 1:]).item() == 0


@pytest.mark.parametrize("shape,prefix", [((16384, 128, 1024), "f32_regtile_splitk4_64x64"),
                                          ((4096, 192, 2000), "f32_regtile_splitk8_64x64"),
                                          ((13000, 130, 2000), "f32_regtile_splitk8_64x96")])
def test_splitk_is_deterministic_and_matches_oracle_at_tall_shape(shape, prefix):
    inp = gi.make_inputs(*shape, dist="uniform", seed=12)
    announce(f"splitk determinism {shape}")
    outs = [run(inp, torch, rt.ALGO_F32_SPLITK).cpu().numpy() for _ in range(3)]
    assert rt.last_kernel().startswith(prefix), rt.last_kernel()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert_parity_sampled(inp, outs[0], f"splitk tall ({rt.last_kernel()})")
