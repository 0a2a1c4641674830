"""Closed-form work and traffic accounting for the kernel ladder (host logic, no GPU).

For a block of outputs computed by one thread with a TM x TN register micro-tile, each k
step loads TM values of A and TN values of B from LDS into registers and performs TM*TN
FMAs ("Understanding Register Tiling" (blog.csdn.net/sweet_ran), the key loop and the
three-version comparison: naive reads 2N values from global memory per output, the
shared-memory kernel reads 2*TILE values from shared memory per output per tile pass and
2N/TILE from global memory, the register-tiled kernel cuts the shared-memory reads per
output by the micro-tile size).

These figures size the roofline terms the benchmark reports: the algorithmic work of a
GEMM is 2*M*N*K flop (the 3*M*N epilogue flops are excluded), and its algorithmic HBM
traffic is one read of A and B, one write of C, plus one read of C when beta != 0.
"""
from __future__ import annotations

from dataclasses import dataclass


def lds_reads_per_fma(tm: int, tn: int) -> float:
    """LDS values read per FMA by a thread with a tm x tn micro-tile: (tm + tn) / (tm * tn)."""
    return (tm + tn) / (tm * tn)


def lds_reads_per_output_per_k(tm: int, tn: int) -> float:
    """Per output element and k step; equal to lds_reads_per_fma (one FMA per output per k)."""
    return lds_reads_per_fma(tm, tn)


def register_loads_per_thread_per_k(tm: int, tn: int) -> int:
    """Values moved from LDS into registers per thread per k step (regA[tm] + regB[tn])."""
    return tm + tn


def lds_read_reduction(tm: int, tn: int) -> float:
    """Factor by which LDS reads fall against one output per thread (2 reads per FMA)."""
    return lds_reads_per_fma(1, 1) / lds_reads_per_fma(tm, tn)


def shared_reads_per_output_per_tile_pass(tile: int) -> int:
    """One output per thread, tile x tile shared tiles: tile reads of sA plus tile of sB."""
    return 2 * tile


def global_reads_per_output_naive(k: int) -> int:
    return 2 * k


def global_reads_per_output_shared(k: int, tile: int) -> float:
    return 2 * k / tile


def block_outputs(threads_x: int, threads_y: int, tm: int, tn: int) -> tuple[int, int]:
    """C block covered by a threads_y x threads_x thread grid with tm x tn micro-tiles."""
    return threads_y * tm, threads_x * tn


def register_estimate(tm: int, tn: int) -> int:
    """Accumulators plus one regA/regB fragment set (addresses and loop state excluded)."""
    return tm * tn + tm + tn


def fmas_per_thread_per_k(tm: int, tn: int) -> int:
    return tm * tn


@dataclass(frozen=True)
class GemmWork:
    M: int
    N: int
    K: int
    elem_bytes_in: int
    beta_nonzero: bool = False

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: A and B read once, C written once (and read if beta != 0)."""
        c = self.M * self.N * 4 * (2 if self.beta_nonzero else 1)
        return (self.M * self.K + self.K * self.N) * self.elem_bytes_in + c

    @property
    def intensity(self) -> float:
        return self.flop / self.hbm_bytes


# MI355X published peaks used as roofline ceilings.
PEAK_FP32_VECTOR_TFLOPS = 157.3  # 256 CU * 2.4 GHz * 256 flop/clk/CU
PEAK_BF16_MFMA_TFLOPS = 2516.6  # dense
PEAK_HBM_GBS = 8000.0
