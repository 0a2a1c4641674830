// regtile_internal.h -- internal interface between the C-ABI front end (regtile_api.hip) and
// the kernel translation units. Not installed; the public interface is include/regtile.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace regtile {

// One validated GEMM problem. Leading dimensions are widened to 64 bits so every offset
// computed from them is 64-bit.
struct Problem {
    int M, N, K;
    float alpha, beta;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    // Storage of the operands (row-major throughout): ta -> A is stored K x M (op(A) is its
    // transpose), tb -> B is stored N x K. The 16-bit entry points' native B is tb.
    bool ta = false, tb = false;
};

// Every launch records the kernel it starts and its workgroup size just before launching it
// (regtile_last_kernel_info queries that kernel's resources).
void note_launch(const void *kernel, unsigned threads);

// A launch reports the kernel it chose through `name` (static storage).
hipError_t launch_scale_c(const Problem &p, hipStream_t s, const char **name);
hipError_t launch_f32_naive(const Problem &p, hipStream_t s, const char **name);
hipError_t launch_f32_lds(const Problem &p, hipStream_t s, const char **name);
hipError_t launch_f32_regtile(const Problem &p, hipStream_t s, const char **name);
hipError_t launch_f32_regtile_small(const Problem &p, hipStream_t s, const char **name);
hipError_t launch_f32_splitk(const Problem &p, hipStream_t s, const char **name);
// 16-bit operand kernels: `f16` selects IEEE fp16 operands, otherwise bf16.
hipError_t launch_bf16_naive(const Problem &p, hipStream_t s, const char **name, bool f16);
// MFMA kernels; `shape` 32 selects 32x32x16 fragments, 16 selects 16x16x32 (on the LDS-DMA
// kernel only; problems it does not take keep the 32x32x16 register-staged kernel).
hipError_t launch_bf16_mfma(const Problem &p, hipStream_t s, const char **name, int shape,
                            bool f16);
// The LDS-DMA kernel's three operand arrangements. Each returns false, launching nothing,
// for a problem it does not take (tile_addressing.h states which it takes); otherwise it
// launches and stores the launch status in *err.
// K-contiguous A and B with 16-byte aligned rows and K a multiple of 8 (M, N and K may end
// inside a tile; 256x256 tiles, or 128x128 up to 128 tiles of 256x256).
bool launch_bf16_mfma_dma(const Problem &p, hipStream_t s, const char **name, int shape, bool f16,
                          hipError_t *err);
// "n n" (A M x K, B K x N, both row-major) or "t t" (A stored K x M, B stored N x K) with K a
// multiple of 8 and the M/N-contiguous operand's column count a multiple of 4.
bool launch_bf16_mfma_dma_rows(const Problem &p, hipStream_t s, const char **name, bool f16,
                               hipError_t *err);
// "t n" (A stored K x M, B stored K x N) with both operands in their own storage in LDS (DMA)
// and transposing fragment reads; M and N multiples of 8, 16-byte aligned rows.
bool launch_bf16_mfma_dma_mn(const Problem &p, hipStream_t s, const char **name, bool f16,
                             hipError_t *err);
// K split over the waves of a workgroup on 64x64 tiles, for problems with few tiles: any of the
// four storage orders, 16-byte aligned rows, within addr::sk_dma_takes.
bool launch_bf16_mfma_splitk(const Problem &p, hipStream_t s, const char **name, bool f16,
                             hipError_t *err);
// The default 16-bit entry points take the split-K kernel for problems of few 64x64 tiles with
// enough K per wave: at most 256 tiles (one per CU) with K >= 1024 in any storage order, and at
// most 512 with K >= 4096 for K-contiguous A and B ("n t") or M/N-contiguous both ("t n").
// Measured against the LDS-DMA kernels (bf16, same box, interleaved, TFLOP/s): "n t" 1024^2 x
// 16384 295 -> 577, 512^2 x 8192 74 -> 163, 1024^2 x 1024 169 -> 193, 1280^2 x 8192 423 ->
// 488; 1024^2 x 16384 "n n" 195 -> 325, "t t" 199 -> 313, "t n" 130 -> 315; 1024 x 2048 x 8192
// "t n" 246 -> 309. Outside the rule: "n t" 1024^2 x 256 70 against 59, 1024 x 2048 x 2048 394
// against 350; 1024 x 2048 x 8192 "n n" 364 against 317, "t t" 367 against 305; 1536^2 x 8192
// (576 tiles) 551 against 450 ("n t").
inline bool bf16_splitk_preferred(const Problem &p) {
    const int64_t t64 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    if (t64 <= 256 && p.K >= 1024) return true;
    return p.ta != p.tb && t64 <= 512 && p.K >= 4096;  // "n t" or "t n"
}

// Host-side launch checks.
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Four consecutive floats at any 4-byte-aligned address as one global_load_dwordx4:
// multi-dword global loads need only dword alignment on gfx9-class GPUs (the compiler emits
// the same single load for this copy).
__device__ __forceinline__ float4 load_f4_any(const float *p) {
    float4 r;
    __builtin_memcpy(&r, p, 16);
    return r;
}

// s_waitcnt lgkmcnt(N) with no wait on the vector-memory or export counters (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}
#define REGTILE_STR2(x) #x
#define REGTILE_STR(x) REGTILE_STR2(x)

// C element update shared by every kernel's epilogue: beta == 0 never reads C.
__device__ __forceinline__ float epilogue_value(float acc, float alpha, float beta,
                                                const float *c) {
    return beta == 0.0f ? alpha * acc : fmaf(alpha, acc, beta * (*c));
}

// The hardware hands out workgroup ids round-robin over the 8 XCDs (id % 8). Renumber so
// that each XCD receives a contiguous run of logical tile ids (neighbouring tiles share A
// rows / B columns in that XCD's L2). Identity when the count is not a multiple of 8.
__device__ __forceinline__ int xcd_contiguous_id(int hw_id, int count) {
    if ((count & 7) != 0) return hw_id;
    return (hw_id & 7) * (count >> 3) + (hw_id >> 3);
}

// Grouped tile order: walk GROUP_M tile-rows at a time, column by column, so consecutive
// logical ids reuse the same B column panel and a small set of A row panels.
template <int GROUP_M>
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per_group = GROUP_M * tiles_n;
    const int group = id / per_group;
    const int first_m = group * GROUP_M;
    const int rows = min(tiles_m - first_m, GROUP_M);
    const int in_group = id - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

}  // namespace regtile
