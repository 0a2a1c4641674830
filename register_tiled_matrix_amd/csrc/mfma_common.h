// mfma_common.h -- device helpers shared by the 16-bit MFMA kernels that stage operands with
// LDS DMA: fragment types, the slab swizzle, the DMA load, counter waits, a barrier that
// waits on nothing, and the two gfx950 MFMA fragment shapes for bf16 and fp16 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_addressing.h"

namespace regtile {
namespace mfma {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// The K-contiguous slab swizzle (tile_addressing.h).
using addr::slab_key;

// One 16-byte-per-lane DMA load: global `src` -> LDS at `dst` + lane * 16 (dst wave-uniform).
// The body exists only in the device pass: the host pass cannot form LDS-space pointers.
__device__ __forceinline__ void dma16(const void *src, void *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
#else
    (void)src;
    (void)dst;
#endif
}

// Buffer descriptor over `bytes` bytes at `base`, raw (untyped) dword access: data format
// 32 in the fourth descriptor word, stride 0 (num_records counts bytes), and the hardware
// returns zero for any byte past num_records. Host-pass stubs exist only to type-check.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
    // The arguments are wave-uniform; readfirstlane states it, so the descriptor lives in
    // scalar registers (a descriptor the compiler believes divergent gets a readfirstlane
    // loop around every load).
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
#else
    (void)base;
    (void)bytes;
    rsrc_t r;
    return r;
#endif
}

// 16 bytes per lane from buffer byte offset voff + soff (soff wave-uniform) into LDS at
// `dst` + lane * 16 (dst wave-uniform): buffer_load_dwordx4 ... lds.
__device__ __forceinline__ void dma16_buf(rsrc_t r, uint32_t voff, uint32_t soff, void *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16,
                                             (int)voff, (int)soff, 0, 0);
#else
    (void)r;
    (void)voff;
    (void)soff;
    (void)dst;
#endif
}

// 8 bytes per lane at buffer byte offset voff + soff (soff wave-uniform); zero past the
// descriptor's end.
__device__ __forceinline__ uint2 load_b64_buf(rsrc_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
#else
    (void)r;
    (void)voff;
    (void)soff;
    return make_uint2(0u, 0u);
#endif
}

// Transposing LDS read (ds_read_b64_tr_b16). Each lane gives the LDS address of 4 consecutive
// 16-bit elements; in every group of 16 lanes, lane 4a + b receives element b of the vectors
// addressed by lanes a, 4 + a, 8 + a and 12 + a (measured). So if lane 4j + a addresses row
// r0 + j, columns c0 + 4a .. c0 + 4a + 3 of a row-major image, lane i receives column c0 + i of
// rows r0 .. r0 + 3.
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const tr_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) tr_v4i16 *)lds);
    return __builtin_bit_cast(uint2, v);
#else
    (void)lds;
    return make_uint2(0u, 0u);
#endif
}

// One fp32 per lane at buffer byte offset voff + soff (soff wave-uniform).
__device__ __forceinline__ float load_f32_buf(rsrc_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
#else
    (void)r;
    (void)voff;
    (void)soff;
    return 0.0f;
#endif
}
__device__ __forceinline__ void store_f32_buf(rsrc_t r, uint32_t voff, uint32_t soff, float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, (int)voff, (int)soff, 0);
#else
    (void)r;
    (void)voff;
    (void)soff;
    (void)x;
#endif
}

// Transpose of a 4 x 8 block of 16-bit values held as 8 runs along the first index: lo[kk] has
// rows 0 and 1 at column kk (row 0 in the low half), hi[kk] rows 2 and 3. out[j] receives row
// j as 8 consecutive columns (dword d = columns 2d, 2d + 1), the form of one 16-byte slab chunk
// of a K-contiguous slab when rows are M (or N) indices and columns are k.
__device__ __forceinline__ void transpose_4x8(const uint32_t lo[8], const uint32_t hi[8], uint4 out[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t *src = j < 2 ? lo : hi;
        uint32_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            d[q] = (j & 1) ? (src[2 * q] >> 16) | (src[2 * q + 1] & 0xFFFF0000u)
                           : (src[2 * q] & 0xFFFFu) | (src[2 * q + 1] << 16);
        out[j] = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

// s_waitcnt lgkmcnt(0) only (LDS reads; LDS DMA is counted by vmcnt, not lgkmcnt).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));

// The two gfx950 MFMA fragment shapes for 16-bit operands (bf16 or fp16, fp32 accumulate).
// Per lane: 8 values of A (row lane % MF, k group lane / MF), 8 values of B (column lane % MF,
// same k group), and MF*MF/64 fp32 accumulators. Fragments are held as raw 16-bit patterns
// (bf16x8) whichever the element type; the fp16 form reinterprets them at the instruction.
//   MF = 32: v_mfma_f32_32x32x16_{bf16,f16}, 16 k per instruction, accumulator v of lane l
//            holds row (v/4)*8 + (l/32)*4 + v%4, column l%32;
//   MF = 16: v_mfma_f32_16x16x32_{bf16,f16}, 32 k per instruction, accumulator v holds row
//            (l/16)*4 + v, column l%16.
// The row splits into a per-lane part (row_lane) and a compile-time per-accumulator part
// (row_acc), so the epilogue's address arithmetic stays constant offsets.
template <int MF, bool F16 = false>
struct Frag;
template <bool F16>
struct Frag<32, F16> {
    typedef f32x16 acc_t;
    static constexpr int KSTEP = 16, NACC = 16;
    __device__ static acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
        if constexpr (F16)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row_lane(int lane) { return addr::c_row_lane<32>(lane); }
    __device__ static constexpr int row_acc(int v) { return addr::c_row_acc<32>(v); }
};
template <bool F16>
struct Frag<16, F16> {
    typedef f32x4 acc_t;
    static constexpr int KSTEP = 32, NACC = 4;
    __device__ static acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
        if constexpr (F16)
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row_lane(int lane) { return addr::c_row_lane<16>(lane); }
    __device__ static constexpr int row_acc(int v) { return addr::c_row_acc<16>(v); }
};

// Workgroup barrier without the memory fence that __syncthreads() adds: the fence makes
// the compiler wait for every outstanding vector-memory operation (vmcnt(0)), which would
// drain the LDS DMA of slabs still in flight. Callers wait for exactly what they need
// (wait_vmcnt / wait_lgkmcnt0) before it. The empty asm statements keep the compiler from
// moving LDS accesses across it; sched_barrier keeps the machine scheduler from doing so.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

}  // namespace mfma
}  // namespace regtile
