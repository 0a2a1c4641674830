"""GPU parity of the operand layouts (BLAS transpose flags over row-major storage).

Every problem is drawn in the oracle's layout (row-major A; row-major B for fp32, column-major
B for bf16/fp16); the device copies are then stored the other way where a test asks for it,
and passed as transposed views. The oracle sees the same values either way.
"""
from __future__ import annotations

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import register_tiled_matrix_amd as rt
from gpu_util import announce, assert_parity_full, assert_parity_sampled, sample_positions

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]  # (trans_a, trans_b): A stored K x M, B stored N x K


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.load()
    yield


def _as(arr, torch_dtype):
    arr = np.ascontiguousarray(arr)
    if torch_dtype == torch.float32:
        return torch.from_numpy(arr).cuda()
    return torch.from_numpy(arr.view(np.int16)).cuda().view(torch_dtype)


def _operands(inp, ta, tb):
    """Device A (M x K) and B (K x N) views with the requested storage; C (row-major)."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[inp.dtype]
    A = _as(inp.A.T, tdt).t() if ta else _as(inp.A, tdt)
    # inp.B is K x N row-major for fp32, N x K (column-major K x N) for the 16-bit types
    if inp.b_col_major:
        B = _as(inp.B, tdt).t() if tb else _as(inp.B.T, tdt)
    else:
        B = _as(inp.B.T, tdt).t() if tb else _as(inp.B, tdt)
    C = (torch.from_numpy(np.ascontiguousarray(inp.C)).cuda() if inp.C is not None
         else torch.empty((inp.M, inp.N), dtype=torch.float32, device="cuda"))
    return A, B, C


def _run(inp, ta, tb, algo=0):
    A, B, C = _operands(inp, ta, tb)
    assert rt._layout(A, "A")[0] == ta and rt._layout(B, "B")[0] == tb
    fn = {"f32": rt.gemm_f32, "bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[inp.dtype]
    fn(A, B, C, alpha=inp.alpha, beta=inp.beta, algo=algo)
    torch.cuda.synchronize()
    return C.cpu().numpy(), rt.last_kernel()


F32_ALGOS = [rt.ALGO_F32_NAIVE, rt.ALGO_F32_REGTILE, rt.ALGO_F32_REGTILE_SMALL, rt.ALGO_F32_AUTO]


@pytest.mark.parametrize("algo", F32_ALGOS)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(1000, 1500, 777), (256, 512, 64), (33, 17, 129)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f32_layouts_full(shape, ta, tb, algo):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype="f32", dist="normal", alpha=1.5, beta=-0.5, seed=M + 3 * N + K)
    announce(f"f32 layout {ta}{tb} {shape} algo={algo}")
    got, name = _run(inp, ta, tb, algo)
    assert_parity_full(inp, got, f"f32 layout ({ta},{tb}) {shape} ({name})")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_f32_layouts_agree_bitwise_with_the_naive_rung(ta, tb):
    # the register-tiled kernels keep fmaf over k in natural order whatever the storage
    inp = gi.make_inputs(300, 260, 333, dtype="f32", dist="normal", seed=41)
    announce(f"f32 layout bitwise {ta}{tb}")
    ref, _ = _run(inp, ta, tb, rt.ALGO_F32_NAIVE)
    for algo in (rt.ALGO_F32_REGTILE, rt.ALGO_F32_REGTILE_SMALL):
        got, name = _run(inp, ta, tb, algo)
        assert np.array_equal(got, ref), name
    nn, _ = _run(inp, 0, 0, rt.ALGO_F32_NAIVE)
    assert np.array_equal(nn, ref)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_f32_layouts_4096_sampled(ta, tb):
    inp = gi.workload_inputs(gi.WORKLOADS["f32_4096"])
    announce(f"f32_4096 layout {ta}{tb}")
    got, name = _run(inp, ta, tb)
    assert "regtile" in name
    assert_parity_sampled(inp, got, f"f32_4096 layout ({ta},{tb}) ({name})")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("algo", [rt.ALGO_BF16_NAIVE, rt.ALGO_BF16_MFMA, rt.ALGO_BF16_AUTO])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(300, 257, 777), (512, 256, 128), (2048, 4096, 192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_16bit_layouts_full(shape, ta, tb, algo, dtype):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=0.5, seed=M + N + 7 * K)
    announce(f"{dtype} layout {ta}{tb} {shape} algo={algo}")
    got, name = _run(inp, ta, tb, algo)
    assert name.startswith(dtype + "_")
    if (ta, tb) == (0, 1) and shape == (2048, 4096, 192) and algo != rt.ALGO_BF16_NAIVE:
        assert "_dma_" in name
    assert_parity_full(inp, got, f"{dtype} layout ({ta},{tb}) {shape} ({name})")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_16bit_layouts_integer_bitwise(ta, tb):
    rng = np.random.Generator(np.random.PCG64(90 + 2 * ta + tb))
    M, N, K = 384, 256, 2048
    A = gi.f32_to_bf16_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
    Bt = gi.f32_to_bf16_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
    inp = gi.GemmInputs(M, N, K, 1.0, 0.0, "bf16", True, A, Bt, None)
    announce(f"bf16 layout integer bitwise {ta}{tb}")
    got, name = _run(inp, ta, tb, rt.ALGO_BF16_MFMA)
    I, J = sample_positions(M, N, seed=6)
    ref, _ = oracle.gemm_inputs_entries(inp, I, J)
    assert np.array_equal(got[I, J].astype(np.float64), ref), name


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (1, 1)])
def test_16bit_layouts_8192_sampled(ta, tb, dtype):
    inp = gi.workload_inputs(gi.WORKLOADS[f"{dtype}_8192"])
    announce(f"{dtype}_8192 layout {ta}{tb}")
    got, name = _run(inp, ta, tb)
    assert_parity_sampled(inp, got, f"{dtype}_8192 layout ({ta},{tb}) ({name})")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", [(4000, 4100, 200), (4001, 4099, 136)], ids=lambda s: "x".join(map(str, s)))
def test_16bit_gathered_layouts_large_ragged(shape, ta, tb, dtype):
    # enough 256x256 tiles for the eight-wave gathered kernel, ragged on every side; the second
    # shape's odd leading dimensions (lda = M for A stored K x M, ldb = N for B stored K x N)
    # make every 8-byte run unaligned. "n n" and "t t" with 8-byte aligned row runs take the
    # DMA kernel instead (the first shape).
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=0.75, beta=0.5, seed=M + N + K + 2 * ta + tb)
    announce(f"{dtype} gathered layout {ta}{tb} {shape}")
    got, name = _run(inp, ta, tb, rt.ALGO_BF16_MFMA)
    rows_dma = ta == tb and K % 8 == 0 and (N if ta == 0 else M) % 4 == 0
    assert ("_dma_" in name) if rows_dma else ("256x256x64_w2x4" in name), name
    assert_parity_sampled(inp, got, f"{dtype} layout ({ta},{tb}) {shape} ({name})")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["integer", "normal"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_16bit_row_operand_on_the_dma_kernel(ta, tb, dtype, dist):
    # "n n" (B stored K x N) and "t t" (A stored K x M) on full tiles (128 of 256x256): the
    # K-contiguous operand over LDS DMA, the other as row runs transposed in registers into the
    # same slabs; integer inputs must match bitwise
    M, N, K = 4096, 2048, 320
    if dist == "integer":
        rng = np.random.Generator(np.random.PCG64(123 + (dtype == "f16")))
        to_bits = gi.f32_to_bf16_bits if dtype == "bf16" else gi.f32_to_f16_bits
        A = to_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
        Bt = to_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
        inp = gi.GemmInputs(M, N, K, 1.0, 0.0, dtype, True, A, Bt, None)
    else:
        inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.0, beta=0.0, seed=321)
    announce(f"{dtype} row operand DMA path {ta}{tb} {dist}")
    got, name = _run(inp, ta, tb, rt.ALGO_BF16_MFMA)
    assert "_dma_" in name and name.endswith("_nn" if ta == 0 else "_tt"), name
    if dist == "integer":
        I, J = sample_positions(M, N, seed=8)
        ref, _ = oracle.gemm_inputs_entries(inp, I, J)
        assert np.array_equal(got[I, J].astype(np.float64), ref), name
    else:
        assert_parity_sampled(inp, got, f"{dtype} row operand ({ta},{tb}) ({name})")


# (the row operand's leading dimension, N for "n n" and M for "t t", a multiple of 4 for its
# 8-byte runs, yet not of 256)
ROWS_RAGGED = [("bf16", 0, 0, (8000, 4100, 1000), "normal"), ("f16", 1, 1, (4100, 8000, 72), "normal"),
               ("bf16", 0, 0, (4097, 8188, 64), "integer"), ("bf16", 1, 1, (4000, 4101, 200), "integer"),
               # at most 128 tiles of 256x256: 128x128 tiles
               ("bf16", 0, 0, (1000, 1500, 776), "normal"), ("f16", 1, 1, (700, 900, 200), "normal"),
               ("bf16", 0, 0, (1536, 1028, 2048), "integer"), ("bf16", 1, 1, (2000, 1001, 520), "integer"),
               ("f16", 0, 0, (33, 4, 8), "normal")]


@pytest.mark.parametrize("dtype,ta,tb,shape,dist", ROWS_RAGGED,
                         ids=[f"{d}-{a}{b}-{'x'.join(map(str, s))}-{t}" for d, a, b, s, t in ROWS_RAGGED])
def test_16bit_row_operand_dma_ragged(dtype, ta, tb, shape, dist):
    # "n n" / "t t" on the DMA kernel with M, N and K ending inside a tile: the row operand's
    # descriptor reads zeros past K; its columns past M / N only feed outputs that are dropped.
    # C has padded rows whose padding must stay untouched.
    M, N, K = shape
    if dist == "integer":
        rng = np.random.Generator(np.random.PCG64(M + N + K))
        to_bits = gi.f32_to_bf16_bits if dtype == "bf16" else gi.f32_to_f16_bits
        A = to_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
        Bt = to_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
        inp = gi.GemmInputs(M, N, K, 1.0, 0.0, dtype, True, A, Bt, None)
    else:
        inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=-0.75, beta=0.5, seed=M + K)
    announce(f"{dtype} row operand DMA ragged {ta}{tb} {shape} {dist}")
    A, B, C0 = _operands(inp, ta, tb)
    big = torch.full((M, N + 5), -77.0, device="cuda")
    C = big[:, :N]
    if inp.C is not None:
        C.copy_(C0)
    fn = {"bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, B, C, alpha=inp.alpha, beta=inp.beta)
    torch.cuda.synchronize()
    name = rt.last_kernel()
    lay = "_nn" if ta == 0 else "_tt"
    assert "_dma_" in name and (name.endswith(lay) or name.endswith(lay + "_ktail")), name
    assert name.endswith("_ktail") == (K % 64 != 0), name
    assert ("_128x128x64_" in name) == (((M + 255) // 256) * ((N + 255) // 256) <= 128), name
    assert torch.all(big[:, N:] == -77.0).item(), "a store landed past column N"
    got = C.cpu().numpy()
    if dist == "integer":
        I, J = sample_positions(M, N, seed=9)
        ref, _ = oracle.gemm_inputs_entries(inp, I, J)
        assert np.array_equal(got[I, J].astype(np.float64), ref), name
    else:
        assert_parity_full(inp, got, f"{dtype} ({ta},{tb}) {shape} ({name})")


TN_DMA = [("bf16", (4096, 2048, 320), "integer", "sampled"), ("f16", (4096, 2048, 320), "normal", "sampled"),
          ("bf16", (4000, 4104, 200), "normal", "full"), ("bf16", (4104, 4000, 1000), "integer", "sampled"),
          ("bf16", (8192, 8192, 8192), "normal", "sampled"),
          # at most 128 tiles of 256x256: 128x128 tiles
          ("bf16", (1000, 1504, 777), "normal", "full"), ("f16", (2048, 2048, 4096), "integer", "sampled"),
          ("bf16", (1536, 1032, 520), "integer", "sampled"), ("f16", (40, 8, 3), "normal", "full")]


@pytest.mark.parametrize("dtype,shape,dist,mode", TN_DMA,
                         ids=[f"{d}-{'x'.join(map(str, s))}-{t}" for d, s, t, _ in TN_DMA])
def test_16bit_tn_on_the_dma_kernel(dtype, shape, dist, mode):
    # "t n" (A stored K x M, B stored K x N): both operands reach LDS by DMA in their own
    # storage and the fragments come from transposing LDS reads; M, N and K may end inside a
    # tile (leading dimensions M and N multiples of 8)
    M, N, K = shape
    if dist == "integer":
        rng = np.random.Generator(np.random.PCG64(M + N + K + 5))
        to_bits = gi.f32_to_bf16_bits if dtype == "bf16" else gi.f32_to_f16_bits
        A = to_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
        Bt = to_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
        inp = gi.GemmInputs(M, N, K, 1.0, 0.0, dtype, True, A, Bt, None)
    else:
        inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=-0.5, seed=M + 3 * N + K)
    announce(f"{dtype} t n DMA {shape} {dist}")
    got, name = _run(inp, 1, 0, rt.ALGO_BF16_MFMA)
    assert "_dma_tr_" in name and (name.endswith("_tn") or name.endswith("_tn_ktail")), name
    assert name.endswith("_ktail") == (K % 64 != 0), name
    assert ("_128x128x64_" in name) == (((M + 255) // 256) * ((N + 255) // 256) <= 128), name
    if dist == "integer":
        I, J = sample_positions(M, N, seed=10)
        ref, _ = oracle.gemm_inputs_entries(inp, I, J)
        assert np.array_equal(got[I, J].astype(np.float64), ref), name
    elif mode == "full":
        assert_parity_full(inp, got, f"{dtype} t n {shape} ({name})")
    else:
        assert_parity_sampled(inp, got, f"{dtype} t n {shape} ({name})")


# M/N-contiguous operands whose column count breaks the descriptor paths' run alignment (a
# multiple of 8 for "t n", of 4 for the row operand of "n n" / "t t"): the DMA launchers refuse
# them, since a run would straddle the descriptor that ends at the operand's last element, and
# the register-staged kernel gathers them, through its per-slab descriptor when the column
# count is a multiple of 4, else through predicated loads.
EDGE_DISPATCH = [("bf16", 1, 0, (1004, 1500, 776)), ("f16", 1, 0, (1001, 1504, 777)),
                 ("bf16", 0, 0, (1000, 1502, 776)), ("bf16", 1, 1, (1002, 1500, 776)),
                 ("f16", 1, 0, (4092, 4100, 512))]


@pytest.mark.parametrize("dtype,ta,tb,shape", EDGE_DISPATCH,
                         ids=[f"{d}-{a}{b}-{'x'.join(map(str, s))}" for d, a, b, s in EDGE_DISPATCH])
def test_16bit_unaligned_column_counts_take_the_staged_gather(dtype, ta, tb, shape):
    M, N, K = shape
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=-0.5, seed=M + 5 * N + K)
    announce(f"{dtype} unaligned column count {ta}{tb} {shape}")
    A, B, C0 = _operands(inp, ta, tb)
    big = torch.full((M, N + 3), -77.0, device="cuda")
    C = big[:, :N]
    C.copy_(C0)
    fn = {"bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[dtype]
    fn(A, B, C, alpha=inp.alpha, beta=inp.beta)
    torch.cuda.synchronize()
    name = rt.last_kernel()
    assert "_dma_" not in name and "_edge" in name, name
    assert torch.all(big[:, N:] == -77.0).item(), "a store landed past column N"
    assert_parity_full(inp, C.cpu().numpy(), f"{dtype} ({ta},{tb}) {shape} ({name})")


# ---- the 16-bit split-K kernel in every storage order ------------------------------------------
# M/N-contiguous operands keep their storage in LDS (64 k-rows of the tile's 64 columns) and
# reach the MFMAs through transposing reads. Shapes: few tiles with deep K, ragged tile edges with
# a K tail (K a multiple of 8 where an operand is K-contiguous), and K below one slab; integer
# inputs compare bitwise, normal inputs within the bound.
SK_LAYOUT_CASES = [((1024, 1024, 2048), "normal"), ((1000, 1000, 776), "normal"), ((72, 136, 72), "normal"),
                   ((512, 256, 4104), "int"), ((64, 64, 8), "normal")]
SK_SUFFIX = {(1, 1): "_tt", (0, 0): "_nn", (1, 0): "_tn", (0, 1): ""}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("case", SK_LAYOUT_CASES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
def test_16bit_splitk_every_layout(case, ta, tb, dtype):
    (M, N, K), dist = case
    if dist == "int":
        rng = np.random.Generator(np.random.PCG64(M + N + K + 2 * ta + tb))
        to_bits = gi.f32_to_bf16_bits if dtype == "bf16" else gi.f32_to_f16_bits
        A = to_bits(rng.integers(-16, 17, M * K).astype(np.float32)).reshape(M, K)
        Bt = to_bits(rng.integers(-16, 17, N * K).astype(np.float32)).reshape(N, K)
        inp = gi.GemmInputs(M, N, K, 1.0, 0.0, dtype, True, A, Bt, None)
    else:
        inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=-0.5, seed=M + N + K + 4 * ta + tb)
    announce(f"{dtype} split-K layout {ta}{tb} {(M, N, K)} {dist}")
    got, name = _run(inp, ta, tb, rt.ALGO_BF16_MFMA_SPLITK)
    ktail = K % 64 != 0 and (ta, tb) != (1, 0)
    assert name == f"{dtype}_mfma32x32x16_splitk4_64x64x64{SK_SUFFIX[(ta, tb)]}" + ("_ktail" if ktail else ""), name
    if dist == "int":
        ref, _ = oracle.gemm_inputs(inp)
        assert np.array_equal(got.astype(np.float64), ref)
    else:
        assert_parity_full(inp, got, f"{dtype} split-K layout ({ta},{tb}) {(M, N, K)} ({name})")
