"""GPU parity for problems with more row blocks than one grid dimension may count in the
one-output-per-thread rungs: the naive rung covers 4 rows per workgroup and the LDS-tiled
rung 32, so these row counts need more than 65536 workgroups down the rows. Both rungs launch a
one-dimensional grid and decode the tile from the workgroup index."""
from __future__ import annotations

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
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,algo,M", [
    ("f32", rt.ALGO_F32_NAIVE, 4 * 65536 + 9),
    ("bf16", rt.ALGO_BF16_NAIVE, 4 * 65536 + 9),
    ("f32", rt.ALGO_F32_LDS, 32 * 65536 + 43),
])
def test_row_blocks_past_65536(dtype, algo, M):
    N, K = 33, 9
    inp = gi.make_inputs(M, N, K, dtype=dtype, dist="normal", alpha=1.25, beta=-0.5, seed=91)
    announce(f"tall grid {dtype} algo={algo} M={M} N={N} K={K}")
    got = run(inp, torch, algo).cpu().numpy()
    name = rt.last_kernel()
    assert name.endswith("naive") or name == "f32_lds_32x32", name
    assert_parity_full(inp, got, f"{dtype} M={M} ({name})")
