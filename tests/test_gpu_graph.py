"""HIP graph capture of the library's launches.

A call makes no allocation, memset or synchronisation: it checks its arguments on the host and
launches one kernel on the caller's stream. So a sequence of calls can be captured into a HIP
graph once and replayed. The test captures a chain that touches each kernel family (split-K on
32x32 and guarded 64x96 tiles, the 128x256 square kernel, the 16-bit LDS-DMA kernel on
128x128 and 256x256 tiles, the 16-bit split-K kernel, beta != 0 calls, and a call that reads
an earlier call's output),
then replays it several times. Between replays the inputs are refreshed in place by eager
work, the same chain runs eagerly into its own outputs, and the device is synchronised. Every
replay must match the eager chain bitwise (the kernels issue a fixed sequence of operations per
output, so the same inputs give the same bits), and the first replay is compared with the fp64
oracle.
"""
from __future__ import annotations

import pytest

import gemm_inputs as gi
import oracle
import register_tiled_matrix_amd as rt
from gpu_util import announce, assert_parity_full, device_operands

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rt.load()
    yield


# (label, dtype, (M, N, K), alpha, beta, algo, kernel name prefix)
CHAIN = [
    ("f32 256^3 split-K", "f32", (256, 256, 256), 1.0, 0.0, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_32x32x16_4x4"),
    ("f32 ragged split-K", "f32", (1000, 1500, 777), 1.5, -0.5, rt.ALGO_F32_AUTO, "f32_regtile_splitk8_64x96x8_8x12_guard"),
    ("f32 square", "f32", (512, 1024, 256), -0.75, 0.0, rt.ALGO_F32_REGTILE, "f32_regtile_128x256x16_8x16"),
    ("bf16 128x128 tiles", "bf16", (2048, 2048, 512), 1.0, 0.5, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_128x128x64"),
    ("bf16 256x256 tiles", "bf16", (4096, 4096, 128), 1.0, 0.0, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_dma_256x256x64"),
    ("bf16 split-K", "bf16", (1024, 1024, 1032), 1.25, -0.5, rt.ALGO_BF16_AUTO, "bf16_mfma32x32x16_splitk4_64x64x64_ktail"),
]


def _host_inputs(version):
    return [gi.make_inputs(M, N, K, dtype=dt, dist="normal", alpha=al, beta=be, seed=1000 * version + i)
            for i, (_, dt, (M, N, K), al, be, _, _) in enumerate(CHAIN)]


def _load(static, inputs):
    """Eager work between replays: copy a new version of every input into the static tensors."""
    for (A, B, C0), inp in zip(static, inputs):
        a, b, c = device_operands(inp, torch)
        A.copy_(a)
        B.copy_(b)
        if inp.C is not None:
            C0.copy_(c)


def _chain(static, outs, tail_out):
    """Run the chain: every call writes its own output; the last call multiplies the first
    output (256 x 256) by itself, so it reads what an earlier call of the same chain wrote."""
    for (A, B, C0), C, (label, dt, _, al, be, algo, _) in zip(static, outs, CHAIN):
        if be != 0.0:
            torch.mul(C0, 1.0, out=C)  # C's start value, by an elementwise kernel in the graph
        fn = rt.gemm_f32 if dt == "f32" else rt.gemm_bf16
        fn(A, B, C, alpha=al, beta=be, algo=algo)
    rt.gemm_f32(outs[0], outs[0], tail_out, alpha=0.5)


def test_graph_replays_match_eager_chain():
    inputs0 = _host_inputs(0)
    static = [device_operands(inp, torch) for inp in inputs0]  # (A, B, initial C) per call
    outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, _, (M, N, _), *_ in CHAIN]
    tail = torch.empty((256, 256), dtype=torch.float32, device="cuda")

    # eager run of the chain, with the kernel each call takes
    announce("graph: eager chain")
    for (A, B, C0), C, (label, dt, _, al, be, algo, prefix) in zip(static, outs, CHAIN):
        if be != 0.0:
            torch.mul(C0, 1.0, out=C)
        (rt.gemm_f32 if dt == "f32" else rt.gemm_bf16)(A, B, C, alpha=al, beta=be, algo=algo)
        torch.cuda.synchronize()
        assert rt.last_kernel().startswith(prefix), (label, rt.last_kernel())

    # warm-up on a side stream, then capture (the binding launches on the current stream,
    # which inside the capture block is the graph's capture stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _chain(static, outs, tail)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("graph: capture")
    with torch.cuda.graph(graph):
        _chain(static, outs, tail)
    torch.cuda.synchronize()

    eager_outs = [torch.empty_like(o) for o in outs]
    eager_tail = torch.empty_like(tail)
    for version in range(4):
        inputs = _host_inputs(version)
        _load(static, inputs)
        torch.cuda.synchronize()
        announce(f"graph: eager chain, version {version}")
        _chain(static, eager_outs, eager_tail)
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        tail.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"graph: replay, version {version}")
        graph.replay()
        torch.cuda.synchronize()
        for o, e, (label, *_rest) in zip(outs, eager_outs, CHAIN):
            assert torch.equal(o, e), f"replay {version}: {label} differs from the eager chain"
        assert torch.equal(tail, eager_tail), f"replay {version}: the dependent call differs"
        if version == 0:
            for o, inp, (label, *_rest) in zip(outs, inputs, CHAIN):
                assert_parity_full(inp, o.cpu().numpy(), f"graph replay: {label}")
            c0 = outs[0].cpu().numpy()
            ref, mag = oracle.gemm(c0, c0, alpha=0.5)
            ok, worst = oracle.check(tail.cpu().numpy(), ref, mag)
            assert ok, f"graph replay: dependent call, worst |err|/bound {worst:.3g}"
