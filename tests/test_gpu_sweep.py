"""GPU determinism and a seeded sweep of edge shapes, against the fp64 oracle.

* Determinism: ten launches of the same problem must give bitwise identical C. The SIMT
  kernels sum every output in a fixed k order and the MFMA kernels issue a fixed sequence of
  instructions per output tile, so a difference between runs could only come from a race
  (an LDS slab overwritten or read before its barrier, a DMA load that lands late).
* Sweep: M, N and K drawn (seeded) from 1, 2, 3, one below / at / above each tile size and
  slab depth, and primes up to 300, on every register-tiled and MFMA rung, each compared in
  full.
"""
from __future__ import annotations

import numpy as np
import pytest

import gemm_inputs as gi
import register_tiled_matrix_amd as rt
from gpu_util import announce, assert_parity_full, run

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.load()
    yield


def _tensor(arr, dtype):
    arr = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(arr).cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(arr.view(np.int16)).cuda().view(tdt)


# (dtype, (M, N, K), trans_a, trans_b, algo, kernel name prefix); 16-bit B is stored N x K
# unless trans_b is 0 (then K x N).
DETERMINISM = [
    ("bf16", (4096, 4096, 4096), 0, 1, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_256x256x64"),
    ("f16", (4096, 4096, 4096), 0, 1, rt.ALGO_BF16_AUTO, "f16_mfma32x32x16_dma_256x256x64"),
    ("bf16", (4096, 4096, 4096), 0, 1, rt.ALGO_BF16_MFMA_16X16, "bf16_mfma16x16x32_dma_256x256x64"),
    ("bf16", (2048, 2048, 4096), 0, 1, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_128x128x64"),
    ("bf16", (4096, 4096, 2048), 1, 0, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_tr_256x256x64"),
    ("bf16", (4096, 4096, 2048), 0, 0, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_256x256x64"),
    ("f16", (4096, 4096, 2048), 1, 1, rt.ALGO_BF16_AUTO, "f16_mfma32x32x16_dma_256x256x64"),
    ("f32", (4096, 4096, 4096), 0, 0, rt.ALGO_F32_AUTO, "f32_regtile_128x256x16_8x16"),
    ("f32", (16384, 128, 4096), 0, 0, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_64x128x8_8x16"),
    ("f32", (1000, 1500, 777), 0, 0, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_64x96x8_8x12"),
    ("f32", (256, 256, 256), 0, 0, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_32x32x16_4x4"),
    ("f32", (1024, 1024, 1024), 0, 0, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_64x64x16_8x8"),
    ("bf16", (1024, 1024, 8192), 0, 1, rt.ALGO_BF16_MFMA_SPLITK, "bf16_mfma32x32x16_splitk4_64x64x64"),
    ("f16", (1000, 1000, 4104), 0, 1, rt.ALGO_BF16_MFMA_SPLITK, "f16_mfma32x32x16_splitk4_64x64x64_ktail"),
]


@pytest.mark.parametrize("dtype,shape,ta,tb,algo,prefix", DETERMINISM,
                         ids=[f"{d}-{'x'.join(map(str, s))}-{a}{b}-{g}" for d, s, a, b, g, _ in DETERMINISM])
def test_ten_runs_are_bitwise_identical(dtype, shape, ta, tb, algo, prefix):
    M, N, K = shape
    rng = np.random.Generator(np.random.PCG64(M + N + K + 10 * ta + tb))
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.standard_normal((K, N), dtype=np.float32)
    if dtype != "f32":
        to_bits = gi.f32_to_bf16_bits if dtype == "bf16" else gi.f32_to_f16_bits
        a = to_bits(a.ravel()).reshape(M, K)
        b = to_bits(b.ravel()).reshape(K, N)
    A = _tensor(a.T, dtype).t() if ta else _tensor(a, dtype)
    B = _tensor(b.T, dtype).t() if tb else _tensor(b, dtype)
    fn = {"f32": rt.gemm_f32, "bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    announce(f"determinism {dtype} {shape} ({ta},{tb}) algo={algo}")
    first = None
    for run_i in range(10):
        C.fill_(float("nan"))
        fn(A, B, C, algo=algo)
        torch.cuda.synchronize()
        assert rt.last_kernel().startswith(prefix), rt.last_kernel()
        if first is None:
            first = C.clone()
            assert torch.isfinite(first).all().item()
        else:
            assert torch.equal(C, first), f"run {run_i} differs from run 0 ({rt.last_kernel()})"


# ---- seeded ragged sweep --------------------------------------------------------------------
PRIMES = [p for p in range(2, 301) if all(p % q for q in range(2, int(p ** 0.5) + 1))]
EDGES = sorted(set([1, 2, 3] + [t + d for t in (8, 16, 32, 64, 128, 256) for d in (-1, 0, 1)] + PRIMES))


def _sweep_shapes(count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [tuple(int(x) for x in rng.choice(EDGES, 3)) for _ in range(count)]


SWEEP = _sweep_shapes(24, 20261202)
F32_RUNGS = [rt.ALGO_F32_AUTO, rt.ALGO_F32_REGTILE, rt.ALGO_F32_SPLITK, rt.ALGO_F32_REGTILE_SMALL]
BF16_RUNGS = [rt.ALGO_BF16_AUTO, rt.ALGO_BF16_MFMA_16X16, rt.ALGO_BF16_MFMA_SPLITK]


@pytest.mark.parametrize("shape", SWEEP, ids=["x".join(map(str, s)) for s in SWEEP])
def test_f32_edge_sweep(shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=1.5, beta=-0.5, seed=M * 31 + N * 7 + K)
    for algo in F32_RUNGS:
        announce(f"f32 sweep {shape} algo={algo}")
        got = run(inp, torch, algo).cpu().numpy()
        assert_parity_full(inp, got, f"f32 sweep {shape} ({rt.last_kernel()})")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SWEEP, ids=["x".join(map(str, s)) for s in SWEEP])
def test_16bit_edge_sweep(shape, dtype):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=-0.75, beta=0.5, seed=M * 29 + N * 5 + K)
    for algo in BF16_RUNGS:
        announce(f"{dtype} sweep {shape} algo={algo}")
        got = run(inp, torch, algo).cpu().numpy()
        assert_parity_full(inp, got, f"{dtype} sweep {shape} ({rt.last_kernel()})")


@pytest.mark.parametrize("shape", SWEEP[:12], ids=["x".join(map(str, s)) for s in SWEEP[:12]])
def test_16bit_edge_sweep_multiples_of_8(shape):
    # the same shapes rounded up to multiples of 8, so that the LDS-DMA kernel (K a multiple
    # of 8, 16-byte aligned rows) takes them rather than the register-staged kernel
    M, N, K = (-(-x // 8) * 8 for x in shape)
    inp = gi.make_inputs(M, N, K, dtype="bf16", dist="normal", alpha=1.25, beta=-0.5, seed=M + N + K)
    announce(f"bf16 sweep x8 {(M, N, K)}")
    got = run(inp, torch, rt.ALGO_BF16_AUTO).cpu().numpy()
    assert "_dma_" in rt.last_kernel(), rt.last_kernel()
    assert_parity_full(inp, got, f"bf16 sweep x8 {(M, N, K)} ({rt.last_kernel()})")
