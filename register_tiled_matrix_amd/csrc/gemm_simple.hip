// gemm_simple.hip -- the lower rungs of the kernel ladder and the scale-only kernel.
//
// Rung 0 (naive) and rung 1 (LDS-tiled) follow the first two versions compared in
// "Understanding Register Tiling" (blog.csdn.net/sweet_ran), section comparing the three
// versions: the naive kernel reads both operands from global memory for every product (2N
// global reads per output), the shared-memory kernel stages 32x32 tiles and still reads
// 32 + 32 = 64 values from LDS per output per tile pass (opening section).
// All rungs accumulate each output with fmaf over k in natural order, so for the same
// inputs they produce bitwise identical results.
#include "regtile_internal.h"

namespace regtile {

// ---------------------------------------------------------------------------------------
// C = beta * C (alpha == 0 or K == 0). beta == 0 writes zeros without reading C.
__global__ __launch_bounds__(256) void scale_c_kernel(int M, int N, float beta, float *C,
                                                      int64_t ldc) {
    const int64_t total = (int64_t)M * N;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / N, j = e - i * N;
        float *c = C + i * ldc + j;
        *c = beta == 0.0f ? 0.0f : beta * (*c);
    }
}

hipError_t launch_scale_c(const Problem &p, hipStream_t s, const char **name) {
    const int64_t total = (int64_t)p.M * p.N;
    const int64_t blocks = (total + 255) / 256;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    note_launch(reinterpret_cast<const void *>(&scale_c_kernel), 256);
    hipLaunchKernelGGL(scale_c_kernel, dim3(grid), dim3(256), 0, s, p.M, p.N, p.beta, p.C, p.ldc);
    *name = "scale_c";
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Rung 0: one thread per output. A workgroup is 4 rows x 64 columns, so each wave64 covers
// 64 consecutive columns of one row: its B reads are one 256-byte run and its A read is a
// broadcast.
template <typename T>
__device__ __forceinline__ float load_as_f32(const T *p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p) {  // bf16 bits
    return __uint_as_float(((uint32_t)(*p)) << 16);
}
template <>
__device__ __forceinline__ float load_as_f32<_Float16>(const _Float16 *p) {  // fp16, exact
    return (float)*p;
}

// TA: A stored K x M (element (i, k) at A[k*lda + i]); TB: B stored N x K (element (k, j) at
// B[j*ldb + k]). Otherwise row-major M x K and K x N.
template <typename T, bool TA, bool TB>
__global__ __launch_bounds__(256) void naive_kernel(int M, int N, int K, float alpha,
                                                    const T *__restrict__ A, int64_t lda,
                                                    const T *__restrict__ B, int64_t ldb,
                                                    float beta, float *__restrict__ C,
                                                    int64_t ldc, int col_blocks) {
    // one-dimensional grid (no 65536 limit on the row blocks): block b covers rows
    // 4 * (b / col_blocks) .. +3 and columns 64 * (b % col_blocks) .. +63
    const int by = blockIdx.x / col_blocks, bx = blockIdx.x - by * col_blocks;
    const int col = bx * 64 + (threadIdx.x & 63);
    const int row = by * 4 + (threadIdx.x >> 6);
    if (row >= M || col >= N) return;
    const T *a = TA ? A + row : A + (int64_t)row * lda;
    const int64_t a_step = TA ? lda : 1;
    const T *b = TB ? B + (int64_t)col * ldb : B + col;
    const int64_t b_step = TB ? 1 : ldb;
    float acc = 0.0f;
    for (int k = 0; k < K; ++k)
        acc = fmaf(load_as_f32(a + k * a_step), load_as_f32(b + k * b_step), acc);
    float *c = C + (int64_t)row * ldc + col;
    *c = epilogue_value(acc, alpha, beta, c);
}

template <typename T>
hipError_t launch_naive(const Problem &p, hipStream_t s) {
    const int col_blocks = (p.N + 63) / 64;
    const int64_t blocks = (int64_t)col_blocks * ((p.M + 3) / 4);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const T *A = (const T *)p.A, *B = (const T *)p.B;
    note_launch(p.ta ? (p.tb ? reinterpret_cast<const void *>(&naive_kernel<T, true, true>)
                             : reinterpret_cast<const void *>(&naive_kernel<T, true, false>))
                     : (p.tb ? reinterpret_cast<const void *>(&naive_kernel<T, false, true>)
                             : reinterpret_cast<const void *>(&naive_kernel<T, false, false>)),
                256);
    if (p.ta && p.tb)
        hipLaunchKernelGGL((naive_kernel<T, true, true>), grid, dim3(256), 0, s, p.M, p.N, p.K,
                           p.alpha, A, p.lda, B, p.ldb, p.beta, p.C, p.ldc, col_blocks);
    else if (p.ta)
        hipLaunchKernelGGL((naive_kernel<T, true, false>), grid, dim3(256), 0, s, p.M, p.N, p.K,
                           p.alpha, A, p.lda, B, p.ldb, p.beta, p.C, p.ldc, col_blocks);
    else if (p.tb)
        hipLaunchKernelGGL((naive_kernel<T, false, true>), grid, dim3(256), 0, s, p.M, p.N, p.K,
                           p.alpha, A, p.lda, B, p.ldb, p.beta, p.C, p.ldc, col_blocks);
    else
        hipLaunchKernelGGL((naive_kernel<T, false, false>), grid, dim3(256), 0, s, p.M, p.N, p.K,
                           p.alpha, A, p.lda, B, p.ldb, p.beta, p.C, p.ldc, col_blocks);
    return hipGetLastError();
}

hipError_t launch_f32_naive(const Problem &p, hipStream_t s, const char **name) {
    *name = "f32_naive";
    return launch_naive<float>(p, s);
}

hipError_t launch_bf16_naive(const Problem &p, hipStream_t s, const char **name, bool f16) {
    *name = f16 ? "f16_naive" : "bf16_naive";
    return f16 ? launch_naive<_Float16>(p, s) : launch_naive<uint16_t>(p, s);
}

// ---------------------------------------------------------------------------------------
// Rung 1: 32x32 tiles in LDS, 1024 threads (16 waves), one output per thread. Each k step
// reads sA[ty][k] (a broadcast within a 32-lane row) and sB[k][tx]. sA rows are padded to
// 33 floats so that the two rows one wave64 touches fall in different banks.
constexpr int LDS_TILE = 32;

__global__ __launch_bounds__(1024) void f32_lds_kernel(int M, int N, int K, float alpha,
                                                       const float *__restrict__ A, int64_t lda,
                                                       const float *__restrict__ B, int64_t ldb,
                                                       float beta, float *__restrict__ C,
                                                       int64_t ldc, int col_blocks) {
    __shared__ float sA[LDS_TILE][LDS_TILE + 1];
    __shared__ float sB[LDS_TILE][LDS_TILE];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    // one-dimensional grid: block b is tile (b / col_blocks, b % col_blocks)
    const int by = blockIdx.x / col_blocks, bx = blockIdx.x - by * col_blocks;
    const int row = by * LDS_TILE + ty;
    const int col = bx * LDS_TILE + tx;
    float acc = 0.0f;
    for (int k0 = 0; k0 < K; k0 += LDS_TILE) {
        sA[ty][tx] = (row < M && k0 + tx < K) ? A[(int64_t)row * lda + k0 + tx] : 0.0f;
        sB[ty][tx] = (k0 + ty < K && col < N) ? B[(int64_t)(k0 + ty) * ldb + col] : 0.0f;
        __syncthreads();
        const int kn = min(LDS_TILE, K - k0);
        if (kn == LDS_TILE) {
#pragma unroll
            for (int k = 0; k < LDS_TILE; ++k) acc = fmaf(sA[ty][k], sB[k][tx], acc);
        } else {
            for (int k = 0; k < kn; ++k) acc = fmaf(sA[ty][k], sB[k][tx], acc);
        }
        __syncthreads();
    }
    if (row < M && col < N) {
        float *c = C + (int64_t)row * ldc + col;
        *c = epilogue_value(acc, alpha, beta, c);
    }
}

hipError_t launch_f32_lds(const Problem &p, hipStream_t s, const char **name) {
    const int col_blocks = (p.N + LDS_TILE - 1) / LDS_TILE;
    const int64_t blocks = (int64_t)col_blocks * ((p.M + LDS_TILE - 1) / LDS_TILE);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    note_launch(reinterpret_cast<const void *>(&f32_lds_kernel), LDS_TILE * LDS_TILE);
    hipLaunchKernelGGL(f32_lds_kernel, dim3((unsigned)blocks), dim3(LDS_TILE * LDS_TILE), 0, s, p.M,
                       p.N, p.K, p.alpha, (const float *)p.A, p.lda, (const float *)p.B, p.ldb,
                       p.beta, p.C, p.ldc, col_blocks);
    *name = "f32_lds_32x32";
    return hipGetLastError();
}

}  // namespace regtile
