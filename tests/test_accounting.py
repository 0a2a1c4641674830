"""Host-side accounting against the numbers the pages print (tests/golden/page_accounting.json)."""
import json
import os

import pytest

from register_tiled_matrix_amd import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_accounting.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["id"] for c in GOLDEN["cases"]])
def test_page_numbers(case):
    got = getattr(acc, case["fn"])(**case["args"])
    want = case["value"]
    if isinstance(want, list):
        assert list(got) == want
    else:
        assert got == pytest.approx(want, rel=0, abs=1e-12)


def test_kernel_configurations_follow_the_accounting():
    # the register-tiled kernel: 8x8 micro-tile -> 0.25 LDS reads per FMA, 8x fewer than
    # one output per thread; the 128x128 tile is 256 threads (4 wave64s)
    assert acc.lds_reads_per_fma(8, 8) == 0.25
    assert acc.lds_read_reduction(8, 8) == 8
    assert acc.block_outputs(16, 16, 8, 8) == (128, 128)
    assert 16 * 16 == 4 * 64


def test_gemm_work():
    w = acc.GemmWork(4096, 4096, 4096, 4)
    assert w.flop == 137438953472
    assert w.hbm_bytes == 3 * 4096 * 4096 * 4
    wb = acc.GemmWork(1000, 1500, 777, 4, beta_nonzero=True)
    assert wb.hbm_bytes == (1000 * 777 + 777 * 1500) * 4 + 2 * 1000 * 1500 * 4
    assert acc.PEAK_FP32_VECTOR_TFLOPS == pytest.approx(256 * 2.4e9 * 256 / 1e12, rel=1e-3)
