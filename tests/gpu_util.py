"""Helpers shared by the GPU tests: move seeded host problems to the device, run one entry
point of the C-ABI library through the binding, and compare with the fp64 oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

import gemm_inputs as gi
import oracle
import register_tiled_matrix_amd as rt


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives output capture)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def device_operands(inp: gi.GemmInputs, torch, device="cuda"):
    """(A, B, C) device tensors in the library's layouts; B is a column-major view for the
    16-bit types (bf16, fp16)."""
    if inp.dtype == "f32":
        A = torch.from_numpy(np.ascontiguousarray(inp.A)).to(device)
        B = torch.from_numpy(np.ascontiguousarray(inp.B)).to(device)
    else:
        tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float16
        A = torch.from_numpy(np.ascontiguousarray(inp.A).view(np.int16)).to(device).view(tdt)
        Bt = torch.from_numpy(np.ascontiguousarray(inp.B).view(np.int16)).to(device).view(tdt)
        B = Bt.t()
    if inp.C is not None:
        C = torch.from_numpy(np.ascontiguousarray(inp.C)).to(device)
    else:
        C = torch.empty((inp.M, inp.N), dtype=torch.float32, device=device)
    return A, B, C


def run(inp: gi.GemmInputs, torch, algo=0, C_init=None):
    """Run the library on `inp`; returns the device C tensor (synchronised)."""
    A, B, C = device_operands(inp, torch)
    if C_init is not None:
        C.copy_(C_init)
    fn = {"f32": rt.gemm_f32, "bf16": rt.gemm_bf16, "f16": rt.gemm_f16}[inp.dtype]
    fn(A, B, C, alpha=inp.alpha, beta=inp.beta, algo=algo)
    torch.cuda.synchronize()
    return C


def assert_parity_full(inp: gi.GemmInputs, got: np.ndarray, what: str = ""):
    ref, mag = oracle.gemm_inputs(inp)
    ok, worst = oracle.check(got, ref, mag)
    assert ok, f"{what}: worst |err|/bound = {worst:.3g}"
    return worst


@functools.lru_cache(maxsize=1)
def workload_reference(name: str):
    """(inputs, ref, mag) of a named workload with the oracle computed over all of C, once per
    process for consecutive uses of the same workload."""
    inp = gi.workload_inputs(gi.WORKLOADS[name])
    ref, mag = oracle.gemm_inputs(inp)
    return inp, ref, mag


def sample_positions(M, N, n_random=65536, seed=0, tile=(256, 256)):
    """Stratified sample of C positions: every (i, j) of the leading tile, every position in
    the last tile row (rows from the last tile boundary to M - 1, all columns) and in the last
    tile column, and n_random seeded uniform positions. Edge tiles are where partial tiles,
    tails and descriptor ends live, so they are covered whole."""
    rng = np.random.Generator(np.random.PCG64(seed))
    tm, tn = min(tile[0], M), min(tile[1], N)
    ii, jj = np.meshgrid(np.arange(tm), np.arange(tn), indexing="ij")
    r0 = ((M - 1) // tile[0]) * tile[0]  # first row of the last tile row
    c0 = ((N - 1) // tile[1]) * tile[1]  # first column of the last tile column
    ri, rj = np.meshgrid(np.arange(r0, M), np.arange(N), indexing="ij")
    ci, cj = np.meshgrid(np.arange(M), np.arange(c0, N), indexing="ij")
    I = [ii.ravel(), ri.ravel(), ci.ravel(), rng.integers(0, M, n_random)]
    J = [jj.ravel(), rj.ravel(), cj.ravel(), rng.integers(0, N, n_random)]
    return np.concatenate(I).astype(np.int64), np.concatenate(J).astype(np.int64)


def assert_parity_sampled(inp: gi.GemmInputs, got: np.ndarray, what: str = "", n_random=65536,
                          seed=0):
    I, J = sample_positions(inp.M, inp.N, n_random=n_random, seed=seed)
    ref, mag = oracle.gemm_inputs_entries(inp, I, J)
    ok, worst = oracle.check(got[I, J], ref, mag)
    assert ok, f"{what}: worst |err|/bound = {worst:.3g} over {len(I)} sampled entries"
    return worst
