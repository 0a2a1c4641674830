/*
 * regtile.h -- C ABI of the register-tiled GEMM library (libregtile.so, gfx950 / MI355X).
 *
 * The library computes dense
 *
 *     C = alpha * A * B + beta * C
 *
 * on one GPU with three levels of tiling: a workgroup tile of C staged from HBM into LDS,
 * and per-thread register micro-tiles of TM x TN accumulators fed by regA/regB fragments
 * at each k step, so that LDS reads per FMA fall by the micro-tile size.
 *   - "Understanding Register Tiling" (blog.csdn.net/sweet_ran, "【infra之路】理解 Register
 *     Tiling"): the shared-memory version (one output per thread), the core idea (a thread
 *     owns a 4x4 block of C), the key loop (regA[TM], regB[TN], TM*TN register FMAs per k)
 *     and the three-version comparison (naive -> shared -> register).
 *   - "寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507), sections 1.1-1.2 (global ->
 *     shared -> register tiling, 128x128 block with 8x8 micro-tiles), section 3 (AMD CDNA:
 *     wave64, VGPR/SGPR split, MFMA fragments) and section 6.3 (register prefetch of the
 *     next k-slice).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: row-major A (M x K, element (i,k) at A[i*lda + k], lda >= max(1,K)) and row-major
 *   C (M x N, element (i,j) at C[i*ldc + j], ldc >= max(1,N)). B is row-major K x N for the
 *   fp32 entry points (B[k*ldb + j], ldb >= max(1,N)) and column-major K x N for the bf16
 *   entry points (B[j*ldb + k], ldb >= max(1,K)).
 * Memory: A, B and C are device pointers owned by the caller (any HIP allocation, e.g. a
 *   PyTorch tensor). The library never allocates, frees or synchronises; it only launches
 *   kernels on `stream` (a hipStream_t; NULL means the default stream). Calls are
 *   asynchronous: C is valid once the stream has been synchronised. Aliasing C with A or
 *   B is not supported.
 * alpha/beta (BLAS convention; the pages compute C = A*B only):
 *   beta == 0  -> C is write-only (its prior contents, NaN included, are never read);
 *   alpha == 0 or K == 0 -> A and B are not read and C = beta * C;
 *   M == 0 or N == 0 -> nothing is launched.
 * Return value: REGTILE_OK (0) on success; -i when argument i (1-based position in the
 *   called function's signature) is invalid -- checked before any HIP call; > 0 is a
 *   hipError_t from the launch. Errors raised while the kernel runs surface at the caller's
 *   next synchronisation, as for any HIP launch.
 * Sizes: M, N, K up to 2^31-1; offsets are computed in 64 bits.
 */
#ifndef REGTILE_H
#define REGTILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REGTILE_OK 0

/* Kernel ladder for the fp32 entry points ("Understanding Register Tiling", the three-version
 * comparison: naive -> shared memory -> register tiling). */
enum regtile_algo_f32 {
    REGTILE_F32_AUTO = 0,    /* library's choice among the register-tiled kernels (3, 4 or 5) */
    REGTILE_F32_NAIVE = 1,   /* one thread per C element, operands straight from HBM */
    REGTILE_F32_LDS = 2,     /* 32x32 LDS tiles, 1024 threads, one C element per thread */
    REGTILE_F32_REGTILE = 3, /* 128x256 LDS tiles, 256 threads, 8x16 register micro-tiles */
    REGTILE_F32_SPLITK = 4,  /* K split over the waves of a workgroup, partials summed in a
                                fixed order (shapes with few tiles): 64x128 (or 64x96) tiles
                                of 8 waves with 8x16 (8x12) micro-tiles, 64x64 tiles of 8 or 4
                                waves with 8x8, or 32x32 tiles of 8 waves with 4x4 */
    REGTILE_F32_REGTILE_SMALL = 5 /* 64x64 tiles, 256 threads, 4x4 register micro-tiles, 4 waves
                                     per SIMD (shapes with few 128x256 tiles) */
};

/* Kernel ladder for the bf16 and fp16 entry points. */
enum regtile_algo_bf16 {
    REGTILE_BF16_AUTO = 0,   /* library's choice: split-K (4) for few tiles, else the MFMA kernel (2) */
    REGTILE_BF16_NAIVE = 1,  /* one thread per C element, fp32 FMA accumulation */
    REGTILE_BF16_MFMA = 2,   /* LDS-tiled, wave-level 32x32x16 MFMA fragments, fp32 accumulators */
    REGTILE_BF16_MFMA_16X16 = 3, /* the same with 16x16x32 fragments where the LDS-DMA kernel
                                    runs 256x256 tiles (other problems as REGTILE_BF16_MFMA):
                                    the shape comparison ("寄存器Tiling跨架构解析" section 3.1) */
    REGTILE_BF16_MFMA_SPLITK = 4 /* K split over the 4 waves of a workgroup on 64x64 tiles,
                                    32x32x16 fragments, partials summed in a fixed order (for
                                    problems with few tiles; "寄存器Tiling跨架构解析" sections 2.4
                                    and 7.2). Any storage order with 16-byte aligned rows: a
                                    K-contiguous operand needs K and its leading dimension
                                    multiples of 8, an M/N-contiguous one its column count and
                                    leading dimension; other problems as REGTILE_BF16_MFMA */
};

/*
 * gemm_f32 -- fp32 C = alpha*A*B + beta*C with fp32 FMA accumulation, on the register-tiled
 * kernel ("Understanding Register Tiling", the key loop; "寄存器Tiling跨架构解析" section 1.1):
 * 128x256 workgroup tiles of 8x16 micro-tiles. Problems with fewer than 384 such tiles (1.5
 * per CU) take smaller tiles (section 2.4 / 7.2 of the second page: tile size against resident
 * waves): with K >= 1024, K >= 384 and fewer than four 64x64 tiles per CU, K >= 128 and fewer
 * than 448 such tiles, or K >= 64 and fewer than 64 of them, the split-K kernel (K split over
 * the waves of a workgroup, 64x128 tiles of 8x16, 64x64 tiles of 8x8 or 32x32 tiles of 4x4
 * micro-tiles, partials summed in a fixed order); otherwise 64x64 tiles of 4x4 micro-tiles at 4
 * waves per SIMD. Every kernel but split-K sums k in natural order, so its results equal the
 * naive rung bitwise; split-K's are deterministic but summed in another order.
 *   M, N, K    (args 1-3)  sizes, >= 0
 *   alpha      (arg 4)     scale of A*B
 *   A, lda     (args 5-6)  device, row-major M x K, lda >= max(1,K); may be NULL if M*K == 0
 *                          or alpha == 0
 *   B, ldb     (args 7-8)  device, row-major K x N, ldb >= max(1,N); NULL allowed as for A
 *   beta       (arg 9)     scale of the prior C
 *   C, ldc     (args 10-11) device, row-major M x N, ldc >= max(1,N); may be NULL if M*N == 0
 *   stream     (arg 12)    hipStream_t or NULL
 */
int gemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, float beta, float *C, int ldc, void *stream);

/*
 * gemm_bf16 -- C = alpha*A*B + beta*C with bf16 operands (raw bit patterns), exact products
 * and fp32 accumulation on CDNA4 MFMA fragments ("寄存器Tiling跨架构解析" section 3.2: MFMA
 * fragments held in VGPRs per lane, accumulators updated in place over k).
 *   A, lda  bf16 row-major M x K (lda >= max(1,K));
 *   B, ldb  bf16 column-major K x N: element (k,j) at B[j*ldb + k] (ldb >= max(1,K));
 *   C, ldc  fp32 row-major M x N.
 * Argument positions and rules as for gemm_f32. Kernel choice: problems of at most 256 tiles of
 * 64x64 with K >= 1024, or at most 512 with K >= 4096 (for this storage order, and for the _ex
 * form's "t n"), take the split-K kernel (REGTILE_BF16_MFMA_SPLITK) when its conditions hold;
 * the rest the MFMA kernels (REGTILE_BF16_MFMA). Both sum each output in a fixed order:
 * repeated calls give identical bits, but the two kernels' roundings differ.
 */
int gemm_bf16(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
              int ldb, float beta, float *C, int ldc, void *stream);

/*
 * gemm_f16 -- C = alpha*A*B + beta*C with IEEE fp16 (binary16) operands given as raw bit
 * patterns, exact products and fp32 accumulation on the same MFMA kernels with
 * v_mfma_f32_32x32x16_f16 fragments: the half-precision GEMM the second page works through
 * ("寄存器Tiling跨架构解析" section 6: fp16 inputs, fp32 accumulation; section 3.2: MFMA
 * fragments). Layouts, argument positions and rules exactly as for gemm_bf16 (A row-major,
 * B column-major, C fp32 row-major).
 */
int gemm_f16(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
             int ldb, float beta, float *C, int ldc, void *stream);

/*
 * regtile_gemm_f32_algo / regtile_gemm_bf16_algo / regtile_gemm_f16_algo -- the same
 * operations on an explicit rung of
 * the kernel ladder (arg 1: a regtile_algo_f32 value, or a regtile_algo_bf16 value for both
 * 16-bit entry points; -1 if unknown). The remaining arguments are those of gemm_f32 /
 * gemm_bf16 / gemm_f16, shifted by one position.
 */
int regtile_gemm_f32_algo(int algo, int M, int N, int K, float alpha, const float *A, int lda,
                          const float *B, int ldb, float beta, float *C, int ldc, void *stream);
int regtile_gemm_bf16_algo(int algo, int M, int N, int K, float alpha, const uint16_t *A,
                           int lda, const uint16_t *B, int ldb, float beta, float *C, int ldc,
                           void *stream);
int regtile_gemm_f16_algo(int algo, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                          const uint16_t *B, int ldb, float beta, float *C, int ldc, void *stream);

/*
 * regtile_gemm_f32_ex / regtile_gemm_bf16_ex / regtile_gemm_f16_ex -- the same products with
 * the storage of each operand chosen (BLAS transpose flags over row-major storage; a step to
 * either side of the pages' row-major kernels):
 *   algo     (arg 1) a regtile_algo_f32 value (fp32) or regtile_algo_bf16 value (16-bit);
 *            -1 if unknown or if that rung stages row-major operands only (the fp32 LDS-tiled
 *            and split-K rungs accept trans_a == trans_b == 0 only)
 *   trans_a  (arg 2) 0: A stored M x K row-major, lda >= max(1,K);
 *                    1: A stored K x M row-major (op(A) is its transpose), lda >= max(1,M)
 *   trans_b  (arg 3) 0: B stored K x N row-major, ldb >= max(1,N);
 *                    1: B stored N x K row-major (column-major K x N), ldb >= max(1,K)
 *   the rest as gemm_f32 / gemm_bf16 / gemm_f16 at positions 4-15; -2 / -3 for a flag other
 *   than 0 or 1. gemm_f32 is (AUTO, 0, 0) and gemm_bf16 / gemm_f16 are (AUTO, 0, 1).
 * Every layout runs on the register-tiled kernels (fp32) or the MFMA kernels (16-bit). The
 * 16-bit LDS-DMA kernel takes (0, 1) whenever K is a multiple of 8 and rows are 16-byte
 * aligned; (0, 0) / (1, 1) when in addition the M- or N-contiguous operand's rows are 8-byte
 * aligned and its leading dimension and column count (N for (0, 0), M for (1, 1)) are
 * multiples of 4 (that operand staged through registers); and (1, 0) with 16-byte aligned
 * rows and M, N, lda and ldb multiples of 8 (both operands in their own storage, transposing
 * LDS reads). Other problems gather M- or N-contiguous operands into K-contiguous LDS slabs
 * with 8-byte loads. No kernel reads or writes outside the caller's matrices: every access
 * stays within the first to last element of A, B and C.
 */
int regtile_gemm_f32_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb, float beta, float *C,
                        int ldc, void *stream);
int regtile_gemm_bf16_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                         const uint16_t *A, int lda, const uint16_t *B, int ldb, float beta,
                         float *C, int ldc, void *stream);
int regtile_gemm_f16_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const uint16_t *A, int lda, const uint16_t *B, int ldb, float beta,
                        float *C, int ldc, void *stream);

/* Name of the kernel the calling thread launched last ("none" before the first launch,
 * "quick-return" when nothing was launched). Static storage; do not free. */
const char *regtile_last_kernel(void);

/*
 * regtile_last_kernel_info -- resources of the kernel the calling thread launched last, as the
 * HIP runtime reports them from its code object (the budget the pages weigh: registers per
 * thread against resident waves, "寄存器Tiling跨架构解析" sections 2.4 and 7.2):
 *   workgroup_size     threads per workgroup;
 *   registers          vector registers per lane (hipFuncAttributes::numRegs);
 *   lds_bytes          static LDS per workgroup;
 *   scratch_bytes      private (spill) memory per lane, 0 when nothing spills;
 *   workgroups_per_cu  resident workgroups per compute unit
 *                      (hipOccupancyMaxActiveBlocksPerMultiprocessor);
 *   waves_per_simd     workgroups_per_cu * workgroup_size / 64 / 4 (4 SIMDs per CU).
 * `info` (arg 1) is caller-owned host memory; -1 if NULL. Returns REGTILE_OK, or a
 * hipError_t (> 0) from the queries; hipErrorInvalidDeviceFunction when this thread has
 * launched no kernel yet (the fields are then 0). Makes no launch and no allocation.
 */
typedef struct regtile_kernel_info {
    int workgroup_size;
    int registers;
    int lds_bytes;
    int scratch_bytes;
    int workgroups_per_cu;
    int waves_per_simd;
} regtile_kernel_info;
int regtile_last_kernel_info(regtile_kernel_info *info);

/* Human-readable text for a status code returned by the entry points. Static storage. */
const char *regtile_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int regtile_version(void);

#ifdef __cplusplus
}
#endif

#endif /* REGTILE_H */
