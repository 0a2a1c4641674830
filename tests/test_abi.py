"""The C-ABI library without a GPU: it loads, exports every symbol include/regtile.h declares,
rejects invalid arguments (LAPACK-style -i) before any HIP call, takes the M == 0 / N == 0
quick return, and every compiled kernel is free of register spills."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import register_tiled_matrix_amd as rt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "regtile.h")


def _ensure_built():
    if not os.path.exists(rt.lib_path()):
        from register_tiled_matrix_amd import build
        build.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    return rt.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert set(names) == set(rt.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rt.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared_functions():
        assert name in exported, f"{name} is not an exported C symbol"


def test_version_and_strerror(lib):
    assert rt.version() == 100
    assert rt.strerror(0) == "success"
    assert "position 6" in rt.strerror(-6)
    assert rt.strerror(1)  # a HIP error string, resolved without a device


DUMMY = 0x1000  # never dereferenced: every call below returns before any HIP call


@pytest.mark.parametrize("args,expect", [
    # M, N, K, alpha, A, lda, B, ldb, beta, C, ldc
    ((-1, 4, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 4), -1),
    ((4, -1, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 4), -2),
    ((4, 4, -1, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 4), -3),
    ((4, 4, 4, 1.0, 0, 4, DUMMY, 4, 0.0, DUMMY, 4), -5),
    ((4, 4, 4, 1.0, DUMMY, 3, DUMMY, 4, 0.0, DUMMY, 4), -6),
    ((4, 4, 4, 1.0, DUMMY, 4, 0, 4, 0.0, DUMMY, 4), -7),
    ((4, 5, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 5), -8),
    ((4, 4, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, 0, 4), -10),
    ((4, 5, 4, 1.0, DUMMY, 4, DUMMY, 5, 0.0, DUMMY, 4), -11),
    ((4, 4, 4, 1.0, DUMMY, 0, DUMMY, 4, 0.0, DUMMY, 4), -6),
])
def test_f32_argument_validation(lib, args, expect):
    assert rt.gemm_f32_raw(*args, 0) == expect
    # the *_algo form shifts every position by one
    assert rt.regtile_gemm_f32_algo(rt.ALGO_F32_REGTILE, *args, 0) == expect - 1


@pytest.mark.parametrize("args,expect", [
    ((4, 4, 6, 1.0, DUMMY, 6, DUMMY, 5, 0.0, DUMMY, 4), -8),   # column-major B: ldb >= K
    ((4, 9, 6, 1.0, DUMMY, 6, DUMMY, 6, 0.0, DUMMY, 8), -11),
    ((4, 4, 6, 1.0, 0, 6, DUMMY, 6, 0.0, DUMMY, 4), -5),
])
def test_bf16_argument_validation(lib, args, expect):
    assert rt.gemm_bf16_raw(*args, 0) == expect
    assert rt.regtile_gemm_bf16_algo(rt.ALGO_BF16_MFMA, *args, 0) == expect - 1
    # fp16 shares the 16-bit layout rules
    assert rt.gemm_f16_raw(*args, 0) == expect
    assert rt.regtile_gemm_f16_algo(rt.ALGO_BF16_MFMA, *args, 0) == expect - 1


def test_unknown_algorithm_is_argument_one(lib):
    a = (4, 4, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 4, 0)
    assert rt.regtile_gemm_f32_algo(6, *a) == -1
    assert rt.regtile_gemm_f32_algo(-1, *a) == -1
    assert rt.regtile_gemm_bf16_algo(5, *a) == -1
    assert rt.regtile_gemm_f16_algo(5, *a) == -1


def test_null_operands_allowed_when_not_read(lib):
    # M == 0: nothing is launched, null pointers are fine
    assert rt.gemm_f32_raw(0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, 0) == 0
    assert rt.last_kernel() == "quick-return"
    assert rt.gemm_bf16_raw(4, 0, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 1, 0) == 0
    assert rt.last_kernel() == "quick-return"


def test_kernel_info_without_a_launch_makes_no_hip_call(lib):
    # NULL -> -1; on a thread that has launched nothing (or whose last call was a quick return)
    # -> hipErrorInvalidDeviceFunction (98), both before any HIP call
    import ctypes
    import threading

    assert lib.regtile_last_kernel_info(None) == -1
    out = {}

    def fresh_thread():
        info = rt.KernelInfo()
        out["fresh"] = lib.regtile_last_kernel_info(ctypes.byref(info))
        rt.gemm_f32_raw(0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, 0)  # quick return
        out["after_quick_return"] = lib.regtile_last_kernel_info(ctypes.byref(info))
        out["fields"] = [getattr(info, n) for n, _ in rt.KernelInfo._fields_]

    t = threading.Thread(target=fresh_thread)
    t.start()
    t.join()
    assert out["fresh"] == 98 and out["after_quick_return"] == 98
    assert out["fields"] == [0] * 6


def test_binding_rejects_host_tensors_and_bad_layouts(lib):
    import torch
    a = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        rt.gemm_f32(a, a)
    with pytest.raises(ValueError):
        rt.gemm_bf16(a.bfloat16(), a.bfloat16())
    with pytest.raises(ValueError):
        rt.gemm_f16(a.half(), a.half())


def test_kernels_have_no_scratch_and_stated_occupancy():
    from register_tiled_matrix_amd import build
    if not os.path.exists(os.path.join(build.BUILD_DIR, "resource_usage.txt")):
        build.build()
    res = build.resource_usage()
    assert res, "no kernel resource remarks were recorded"
    for name, r in res.items():
        assert r.get("ScratchSize [bytes/lane]", 0) == 0, (name, r)
    f32 = [r for n, r in res.items() if "f32_regtile_kernel" in n]
    assert f32 and all(r["Occupancy [waves/SIMD]"] >= 2 for r in f32)
    small = [r for n, r in res.items() if "f32_regtile_kernel" in n and "SmallCfg" in n]
    assert small and all(r["Occupancy [waves/SIMD]"] >= 4 for r in small)
    assert all(r["VGPRs"] + r.get("AGPRs", 0) <= 512 // r["Occupancy [waves/SIMD]"] for r in f32)


@pytest.mark.parametrize("fn", ["regtile_gemm_f32_ex", "regtile_gemm_bf16_ex", "regtile_gemm_f16_ex"])
def test_layout_entry_points_validate_flags_and_leading_dimensions(lib, fn):
    f = getattr(rt, fn)
    # algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream
    base = dict(algo=0, ta=0, tb=0, M=4, N=5, K=6, lda=6, ldb=5, ldc=5)

    def call(**kw):
        a = {**base, **kw}
        return f(a["algo"], a["ta"], a["tb"], a["M"], a["N"], a["K"], 1.0, DUMMY, a["lda"], DUMMY,
                 a["ldb"], 0.0, DUMMY, a["ldc"], 0)

    assert call(ta=2) == -2 and call(tb=-1) == -3
    assert call(M=-1) == -4 and call(N=-1) == -5 and call(K=-1) == -6
    assert call(lda=5) == -9            # A stored M x K: lda >= K
    assert call(ta=1, lda=3) == -9      # A stored K x M: lda >= M
    assert call(ldb=4) == -11           # B stored K x N: ldb >= N
    assert call(tb=1, ldb=5) == -11     # B stored N x K: ldb >= K
    assert call(ldc=4) == -14
    assert call(algo=9) == -1
    assert call(M=0) == 0 and rt.last_kernel() == "quick-return"


def test_row_major_only_rungs_reject_transposed_layouts(lib):
    a = (4, 4, 4, 1.0, DUMMY, 4, DUMMY, 4, 0.0, DUMMY, 4, 0)
    for algo in (rt.ALGO_F32_LDS, rt.ALGO_F32_SPLITK):
        assert rt.regtile_gemm_f32_ex(algo, 1, 0, *a) == -1
        assert rt.regtile_gemm_f32_ex(algo, 0, 1, *a) == -1

