"""The blocked CPU baseline GEMM agrees with the fp64 oracle (it is timed next to the GPU)."""
import numpy as np
import pytest

import cpu_baseline
import gemm_inputs as gi
import oracle


@pytest.mark.parametrize("M,N,K,alpha,beta", [(1, 1, 1, 1.0, 0.0), (37, 53, 300, 1.5, -0.5),
                                              (129, 2100, 257, 1.0, 0.0), (300, 17, 1000, -2.0, 1.0),
                                              (256, 256, 256, 1.0, 0.0), (5, 7, 0, 1.0, 2.0)])
def test_blocked_matches_oracle(M, N, K, alpha, beta):
    inp = gi.make_inputs(M, N, K, dist="normal", alpha=alpha, beta=beta, seed=M + N + K, with_c=True)
    got = cpu_baseline.sgemm(inp.A, inp.B, inp.C.copy(), alpha=alpha, beta=beta)
    ref, mag = oracle.gemm(inp.A, inp.B, inp.C, alpha=alpha, beta=beta)
    ok, worst = oracle.check(got, ref, mag)
    assert ok, worst


def test_blocked_integer_exact():
    rng = np.random.Generator(np.random.PCG64(3))
    A = rng.integers(-16, 17, (200, 300)).astype(np.float32)
    B = rng.integers(-16, 17, (300, 150)).astype(np.float32)
    got = cpu_baseline.sgemm(A, B)
    assert np.array_equal(got.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64))
