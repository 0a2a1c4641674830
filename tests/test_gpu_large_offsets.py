"""GPU parity with leading dimensions so large that row offsets pass 2^31 bytes.

The kernels take int64 leading dimensions and form every element offset in 64 bits; the LDS-DMA
bf16/fp16 kernel addresses a tile through 32-bit buffer offsets and is eligible only while a
tile's rows span less than 2^31 bytes, so these problems must fall back to the register-staged
kernel. Only the leading M x K / K x N / M x N corner of each allocation is written or read.
"""
from __future__ import annotations

import numpy as np
import pytest

import gemm_inputs as gi
import register_tiled_matrix_amd as rt
from gpu_util import announce, assert_parity_full, assert_parity_sampled

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GIB = 1 << 30


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.load()
    yield
    torch.cuda.empty_cache()


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes + 4 * GIB:
        pytest.skip(f"needs {nbytes / GIB:.0f} GiB of free device memory")


def _strided(rows, cols, ld, dtype, host=None):
    """A rows x cols view with row stride `ld` into a rows x ld allocation (uninitialised
    outside the view); `host` (numpy, rows x cols; raw 16-bit patterns for bf16/fp16) is copied
    in when given."""
    view = torch.empty((rows, ld), dtype=dtype, device="cuda")[:, :cols]
    if host is not None:
        h = np.ascontiguousarray(host)
        src = torch.from_numpy(h) if dtype == torch.float32 else torch.from_numpy(h.view(np.int16)).view(dtype)
        view.copy_(src.cuda())
    return view


F32_ALGOS = [rt.ALGO_F32_NAIVE, rt.ALGO_F32_LDS, rt.ALGO_F32_REGTILE, rt.ALGO_F32_REGTILE_SMALL,
             rt.ALGO_F32_SPLITK, rt.ALGO_F32_AUTO]


@pytest.fixture(scope="module")
def f32_problem():
    M, N, K = 300, 260, 100
    lda, ldb, ldc = 1_800_000, 5_500_000, 1_800_000  # multiples of 8: vector paths stay on
    assert (M - 1) * lda * 4 >= 2**31 and (K - 1) * ldb * 4 >= 2**31 and (M - 1) * ldc * 4 >= 2**31
    _need((M * lda + K * ldb + M * ldc) * 4)
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=1.5, beta=-0.5, seed=77)
    A = _strided(M, K, lda, torch.float32, inp.A)
    B = _strided(K, N, ldb, torch.float32, inp.B)
    C = _strided(M, N, ldc, torch.float32)
    yield inp, A, B, C
    del A, B, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", F32_ALGOS)
def test_f32_leading_dimensions_past_2gib(f32_problem, algo):
    inp, A, B, C = f32_problem
    assert rt._layout(A, "A") == (0, A.stride(0)) and A.stride(0) == 1_800_000
    C.copy_(torch.from_numpy(inp.C).cuda())
    announce(f"f32 large leading dimensions algo={algo}")
    rt.gemm_f32(A, B, C, alpha=inp.alpha, beta=inp.beta, algo=algo)
    torch.cuda.synchronize()
    assert_parity_full(inp, C.cpu().numpy(), f"f32 lda/ldb/ldc past 2 GiB, algo {algo} ({rt.last_kernel()})")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_tile_offsets_past_32_bits_fall_back_to_the_staged_kernel(dtype):
    # 256 full 256x256 tiles would take the LDS-DMA kernel, but 256 rows of A (and of C) span
    # more than 2^31 bytes, beyond its 32-bit buffer offsets.
    M, N, K = 4096, 4096, 64
    lda, ldc = 4_194_312, 2_097_160
    assert 256 * lda * 2 >= 2**31 and 256 * ldc * 4 >= 2**31
    _need(M * lda * 2 + M * ldc * 4)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", seed=78)
    A = _strided(M, K, lda, tdt, inp.A)
    Bt = torch.from_numpy(inp.B.view(np.int16)).cuda().view(tdt)  # N x K, K-contiguous
    C = _strided(M, N, ldc, torch.float32)
    announce(f"{dtype} large lda/ldc")
    fn = {"bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, Bt.t(), C)
    torch.cuda.synchronize()
    name = rt.last_kernel()
    assert "_dma_" not in name and name.startswith(dtype + "_mfma_256x256"), name
    got = C.cpu().numpy()
    del A, C
    torch.cuda.empty_cache()
    assert_parity_sampled(inp, got, f"{dtype} lda/ldc past 32-bit tile offsets ({name})")
    # with compact strides the same problem takes the LDS-DMA kernel
    A2 = torch.from_numpy(inp.A.view(np.int16)).cuda().view(tdt)
    C2 = fn(A2, Bt.t())
    torch.cuda.synchronize()
    assert "_dma_" in rt.last_kernel()
    assert_parity_sampled(inp, C2.cpu().numpy(), f"{dtype} compact strides ({rt.last_kernel()})")
