"""register_tiled_matrix_amd -- register-tiled GEMM for MI355X (gfx950), Python binding.

A thin ctypes binding over the C ABI of ``libregtile.so`` (declared in ``include/regtile.h``).
It only marshals arguments: every step of the product runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.

Entry points (same names as the C ABI):

* ``gemm_f32(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_F32_AUTO)``
  fp32 ``C = alpha*A@B + beta*C``; A (M x K) and B (K x N) row-major fp32 CUDA tensors
  (row stride may exceed the width), C (M x N) row-major fp32.
* ``gemm_bf16(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_BF16_AUTO)``
  bf16 A (M x K) times bf16 B (K x N), fp32 C; the fast path is row-major A with B given as a
  column-major view (for example ``Bt.t()`` for a contiguous N x K tensor ``Bt``).
* Every tensor entry point accepts A and B either row-major or as transposed (column-major)
  views and passes the layout to the ``regtile_gemm_*_ex`` entry points.
* ``gemm_f16(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_BF16_AUTO)`` the same with
  float16 A and B (IEEE binary16); the algorithm values are the bf16 ones.
* ``gemm_f32_raw`` / ``gemm_bf16_raw`` / ``gemm_f16_raw`` take the C arguments verbatim
  (integers for pointers).
* ``last_kernel()``, ``last_kernel_info()`` (registers, LDS, scratch and occupancy of that
  kernel, from the HIP runtime), ``strerror(status)``, ``version()``.

The library must be built (``python -m register_tiled_matrix_amd.build``); importing this
package does not build it, and every call raises ``RegtileLibraryMissing`` when it is absent.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "ALGO_F32_AUTO", "ALGO_F32_NAIVE", "ALGO_F32_LDS", "ALGO_F32_REGTILE", "ALGO_F32_SPLITK",
    "ALGO_F32_REGTILE_SMALL",
    "ALGO_BF16_AUTO", "ALGO_BF16_NAIVE", "ALGO_BF16_MFMA", "ALGO_BF16_MFMA_16X16", "ALGO_BF16_MFMA_SPLITK",
    "RegtileError", "RegtileLibraryMissing", "lib_path", "load",
    "gemm_f32", "gemm_bf16", "gemm_f16", "gemm_f32_raw", "gemm_bf16_raw", "gemm_f16_raw",
    "regtile_gemm_f32_algo", "regtile_gemm_bf16_algo", "regtile_gemm_f16_algo",
    "regtile_gemm_f32_ex", "regtile_gemm_bf16_ex", "regtile_gemm_f16_ex",
    "last_kernel", "last_kernel_info", "strerror", "version", "EXPORTED_SYMBOLS",
]

ALGO_F32_AUTO, ALGO_F32_NAIVE, ALGO_F32_LDS, ALGO_F32_REGTILE, ALGO_F32_SPLITK = 0, 1, 2, 3, 4
ALGO_F32_REGTILE_SMALL = 5
ALGO_BF16_AUTO, ALGO_BF16_NAIVE, ALGO_BF16_MFMA, ALGO_BF16_MFMA_16X16, ALGO_BF16_MFMA_SPLITK = 0, 1, 2, 3, 4

EXPORTED_SYMBOLS = ("gemm_f32", "gemm_bf16", "gemm_f16", "regtile_gemm_f32_algo",
                    "regtile_gemm_bf16_algo", "regtile_gemm_f16_algo", "regtile_gemm_f32_ex",
                    "regtile_gemm_bf16_ex", "regtile_gemm_f16_ex",
                    "regtile_last_kernel", "regtile_last_kernel_info", "regtile_strerror",
                    "regtile_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libregtile.so")
_lib = None
_lock = threading.Lock()


class KernelInfo(ctypes.Structure):
    """regtile_kernel_info of include/regtile.h."""
    _fields_ = [("workgroup_size", ctypes.c_int), ("registers", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("scratch_bytes", ctypes.c_int), ("workgroups_per_cu", ctypes.c_int),
                ("waves_per_simd", ctypes.c_int)]


class RegtileError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"regtile status {status}: {message}")
        self.status = status


class RegtileLibraryMissing(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libregtile.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RegtileLibraryMissing(
                f"{_LIB_PATH} is not built; run `python -m register_tiled_matrix_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        I, F, P = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        gemm = [I, I, I, F, P, I, P, I, F, P, I, P]
        for name, args in (("gemm_f32", gemm), ("gemm_bf16", gemm), ("gemm_f16", gemm),
                           ("regtile_gemm_f16_algo", [I] + gemm),
                           ("regtile_gemm_f32_ex", [I, I, I] + gemm),
                           ("regtile_gemm_bf16_ex", [I, I, I] + gemm),
                           ("regtile_gemm_f16_ex", [I, I, I] + gemm),
                           ("regtile_gemm_f32_algo", [I] + gemm),
                           ("regtile_gemm_bf16_algo", [I] + gemm)):
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = I
        lib.regtile_last_kernel.argtypes = []
        lib.regtile_last_kernel.restype = ctypes.c_char_p
        lib.regtile_last_kernel_info.argtypes = [ctypes.POINTER(KernelInfo)]
        lib.regtile_last_kernel_info.restype = I
        lib.regtile_strerror.argtypes = [I]
        lib.regtile_strerror.restype = ctypes.c_char_p
        lib.regtile_version.argtypes = []
        lib.regtile_version.restype = I
        _lib = lib
        return lib


def last_kernel() -> str:
    return load().regtile_last_kernel().decode()


def last_kernel_info() -> dict:
    """Resources of the kernel this thread launched last (regtile_last_kernel_info)."""
    info = KernelInfo()
    _check(load().regtile_last_kernel_info(ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in KernelInfo._fields_}


def strerror(status: int) -> str:
    return load().regtile_strerror(int(status)).decode()


def version() -> int:
    return int(load().regtile_version())


def _check(status: int) -> None:
    if status != 0:
        raise RegtileError(status, strerror(status))


# ---- raw entry points: the C arguments verbatim -------------------------------------------
def gemm_f32_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_bf16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def regtile_gemm_f32_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().regtile_gemm_f32_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                        stream)


def gemm_f16_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def regtile_gemm_f16_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().regtile_gemm_f16_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                        stream)


def regtile_gemm_f32_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        stream=0) -> int:
    return load().regtile_gemm_f32_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb,
                                      beta, C, ldc, stream)


def regtile_gemm_bf16_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=0) -> int:
    return load().regtile_gemm_bf16_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb,
                                       beta, C, ldc, stream)


def regtile_gemm_f16_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        stream=0) -> int:
    return load().regtile_gemm_f16_ex(algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb,
                                      beta, C, ldc, stream)


def regtile_gemm_bf16_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().regtile_gemm_bf16_algo(algo, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                         stream)


# ---- tensor entry points -------------------------------------------------------------------
def _stream_handle(t, stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _row_major_ld(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (unit column stride)")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows overlap (row stride below the width)")
    return max(int(t.stride(0)), int(t.shape[1]), 1)


def _layout(t, name):
    """(trans, ld) of a 2-D operand: row-major storage (unit column stride) -> (0, row stride);
    column-major storage (unit row stride), i.e. the transpose of a row-major matrix ->
    (1, column stride). Anything else (overlapping or non-unit strides) is rejected."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    r, c = t.shape
    if (c <= 1 or t.stride(1) == 1) and (r <= 1 or t.stride(0) >= c):
        return 0, max(int(t.stride(0)), int(c), 1)
    if (r <= 1 or t.stride(0) == 1) and (c <= 1 or t.stride(1) >= r):
        return 1, max(int(t.stride(1)), int(r), 1)
    raise ValueError(f"{name} must be row-major or column-major with non-overlapping rows")


def _out(C, M, N, like):
    import torch

    if C is None:
        return torch.empty((M, N), dtype=torch.float32, device=like.device)
    if C.dtype != torch.float32 or tuple(C.shape) != (M, N):
        raise ValueError(f"C must be float32 of shape {(M, N)}")
    return C


def _gemm(fn, want, label, A, B, C, alpha, beta, algo, stream):
    if A.dtype != want or B.dtype != want:
        raise ValueError(f"{label} takes {want} A and B")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError(f"{label} takes device tensors")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if C is None and beta != 0.0:
        raise ValueError("beta != 0 needs C")
    C = _out(C, M, N, A)
    (ta, lda), (tb, ldb) = _layout(A, "A"), _layout(B, "B")
    ldc = _row_major_ld(C, "C")
    st = fn(int(algo), ta, tb, M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
            float(beta), C.data_ptr(), ldc, _stream_handle(A, stream))
    _check(st)
    return C


def gemm_f32(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_F32_AUTO, stream=None):
    """C = alpha*A@B + beta*C on fp32 CUDA tensors; returns C (allocated when None). A and B
    may each be row-major or a transposed (column-major) view; C is row-major."""
    import torch

    return _gemm(regtile_gemm_f32_ex, torch.float32, "gemm_f32", A, B, C, alpha, beta, algo,
                 stream)


def gemm_bf16(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_BF16_AUTO, stream=None):
    """C = alpha*A@B + beta*C; bf16 A (M x K) and B (K x N), each row-major or a transposed
    view (the fast path is row-major A with column-major B, e.g. ``Bt.t()``), fp32 C row-major;
    returns C (allocated when None)."""
    import torch

    return _gemm(regtile_gemm_bf16_ex, torch.bfloat16, "gemm_bf16", A, B, C, alpha, beta, algo,
                 stream)


def gemm_f16(A, B, C=None, alpha=1.0, beta=0.0, algo=ALGO_BF16_AUTO, stream=None):
    """As gemm_bf16 with float16 (IEEE binary16) A and B."""
    import torch

    return _gemm(regtile_gemm_f16_ex, torch.float16, "gemm_f16", A, B, C, alpha, beta, algo,
                 stream)
