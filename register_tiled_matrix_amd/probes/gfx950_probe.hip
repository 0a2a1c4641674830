// gfx950_probe.hip -- small measurements of the gfx950 facts the kernels are designed around.
// Not part of the library: `python -m register_tiled_matrix_amd.tune probe` builds this file
// with the library's compiler flags and runs it.
//
//   valu  FP32 FMA issue rate (non-packed v_fmac_f32, VGPR operands) at 1, 2 and 4 waves per
//         SIMD, and the effect of VGPR banks (register number mod 4): accumulator and src0 in
//         one bank, accumulator and src1 in one bank, neither, all three operands in even
//         banks. Each wave also reports its own
//         shader-clock cycles (s_memtime) against the constant-rate wall clock, which gives
//         the clock the SIMD ran at and the cycles one wave64 FMA took per SIMD.
//   mfma  v_mfma_f32_32x32x16_bf16 with 8 independent accumulators per wave: the attainable
//         matrix rate on this machine.
//   valu_sustained  FP32 FMAs at two waves per SIMD for 30 back-to-back launches of a few ms,
//         with constant and with random operands.
//   mfma_sustained  the MFMA loop for 30 back-to-back launches of a few ms, with constant and with
//         random bf16 operands: the clock the package sustains under matrix load alone.
//   lds_tr  the lane mapping of ds_read_b64_tr_b16 (transposing 16-bit LDS read).
//   lds   one kernel per LDS address pattern (16 bytes per lane); run under
//         `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVES` for the
//         cycles and conflict cycles per instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);          \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

// ---- valu ---------------------------------------------------------------------------------
// 16 FMAs into accumulators v32, v36, ..., v92 (all in bank 0) with the given sources.
#define FMA1(D, S0, S1) "v_fmac_f32 " D ", " S0 ", " S1 "\n"
#define FMA16(S0, S1)                                                                      \
    FMA1("v32", S0, S1) FMA1("v36", S0, S1) FMA1("v40", S0, S1) FMA1("v44", S0, S1)       \
    FMA1("v48", S0, S1) FMA1("v52", S0, S1) FMA1("v56", S0, S1) FMA1("v60", S0, S1)       \
    FMA1("v64", S0, S1) FMA1("v68", S0, S1) FMA1("v72", S0, S1) FMA1("v76", S0, S1)       \
    FMA1("v80", S0, S1) FMA1("v84", S0, S1) FMA1("v88", S0, S1) FMA1("v92", S0, S1)
#define VALU_CLOBBERS                                                                      \
    "v1", "v2", "v4", "v32", "v36", "v40", "v44", "v48", "v52", "v56", "v60", "v64", "v68", \
        "v72", "v76", "v80", "v84", "v88", "v92"
#define VALU_INIT                                                                          \
    "v_mov_b32 v1, 1.0\nv_mov_b32 v2, 1.0\nv_mov_b32 v4, 1.0\n"                            \
    "v_mov_b32 v32, 0\nv_mov_b32 v36, 0\nv_mov_b32 v40, 0\nv_mov_b32 v44, 0\n"             \
    "v_mov_b32 v48, 0\nv_mov_b32 v52, 0\nv_mov_b32 v56, 0\nv_mov_b32 v60, 0\n"             \
    "v_mov_b32 v64, 0\nv_mov_b32 v68, 0\nv_mov_b32 v72, 0\nv_mov_b32 v76, 0\n"             \
    "v_mov_b32 v80, 0\nv_mov_b32 v84, 0\nv_mov_b32 v88, 0\nv_mov_b32 v92, 0\n"

constexpr int kValuIters = 2000, kValuFmaPerIter = 64;

// P = 0: src0 v1, src1 v2 (no operand shares the accumulators' bank)
// P = 1: src0 v4, src1 v1 (accumulator and src0 in bank 0)
// P = 2: src0 v1, src1 v4 (accumulator and src1 in bank 0)
// P = 3: src0 v4, src1 v2 (accumulator, src0 and src1 all in even banks)
template <int P>
__global__ __launch_bounds__(256) void valu_kernel(uint64_t *out, int iters) {
    asm volatile(VALU_INIT ::: VALU_CLOBBERS);
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
        if (P == 0) asm volatile(FMA16("v1", "v2") FMA16("v1", "v2") FMA16("v1", "v2") FMA16("v1", "v2") ::: VALU_CLOBBERS);
        if (P == 1) asm volatile(FMA16("v4", "v1") FMA16("v4", "v1") FMA16("v4", "v1") FMA16("v4", "v1") ::: VALU_CLOBBERS);
        if (P == 2) asm volatile(FMA16("v1", "v4") FMA16("v1", "v4") FMA16("v1", "v4") FMA16("v1", "v4") ::: VALU_CLOBBERS);
        if (P == 3) asm volatile(FMA16("v4", "v2") FMA16("v4", "v2") FMA16("v4", "v2") FMA16("v4", "v2") ::: VALU_CLOBBERS);
    }
    const uint64_t t1 = clock64(), w1 = wall_clock64();
    if ((threadIdx.x & 63) == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        out[2 * w] = t1 - t0;
        out[2 * w + 1] = w1 - w0;
    }
}

int run_valu() {
    const int max_blocks = 256 * 4;
    uint64_t *d;
    CHECK(hipMalloc(&d, sizeof(uint64_t) * 2 * 4 * max_blocks));
    static uint64_t h[2 * 4 * 256 * 4];
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    typedef void (*kfn)(uint64_t *, int);
    const struct { const char *name; kfn fn; } pats[] = {
        {"no shared bank", valu_kernel<0>}, {"acc + src0 bank", valu_kernel<1>}, {"acc + src1 bank", valu_kernel<2>},
        {"all three in even banks", valu_kernel<3>}};
    printf("| operands | waves/SIMD | SIMD cycles per wave64 FMA | clock GHz | TFLOP/s |\n|---|---|---|---|---|\n");
    for (int per_simd = 1; per_simd <= 4; per_simd *= 2)
        for (const auto &p : pats) {
            const int blocks = 256 * per_simd;  // 256 threads = one wave per SIMD of a CU
            hipLaunchKernelGGL(p.fn, dim3(blocks), dim3(256), 0, 0, d, kValuIters);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e0));
            hipLaunchKernelGGL(p.fn, dim3(blocks), dim3(256), 0, 0, d, kValuIters);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            CHECK(hipMemcpy(h, d, sizeof(uint64_t) * 2 * 4 * blocks, hipMemcpyDeviceToHost));
            double cyc = 0, wall = 0;
            for (int i = 0; i < 4 * blocks; ++i) {
                cyc += (double)h[2 * i];
                wall += (double)h[2 * i + 1];
            }
            cyc /= 4 * blocks;
            wall /= 4 * blocks;
            const double fmas = (double)kValuIters * kValuFmaPerIter;
            const double ghz = cyc / (wall / (wall_khz * 1e3)) / 1e9;
            const double tflops = 2.0 * fmas * 64 * 4 * blocks / (ms * 1e-3) / 1e12;
            printf("| %s | %d | %.2f | %.2f | %.1f |\n", p.name, per_simd, cyc / fmas / per_simd, ghz, tflops);
        }
    return 0;
}

// ---- mfma ---------------------------------------------------------------------------------
typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__global__ __launch_bounds__(256) void mfma_kernel(float *out, uint64_t *clk, int iters) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (short)(0x3f80 + (threadIdx.x & 7));  // bf16 values near 1
        b[i] = (short)(0x3c00 + i);                  // small bf16 values
    }
    f32x16 acc[8];
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    const uint64_t t1 = clock64(), w1 = wall_clock64();
    if ((threadIdx.x & 63) == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = w1 - w0;
    }
    float s = 0.0f;
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

int run_mfma() {
    const int blocks = 256, iters = 4000;
    float *d;
    uint64_t *clk;
    CHECK(hipMalloc(&d, sizeof(float) * blocks * 256));
    CHECK(hipMalloc(&clk, sizeof(uint64_t) * 2 * 4 * blocks));
    static uint64_t h[2 * 4 * 256];
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, 0, d, clk, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, 0, d, clk, iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipMemcpy(h, clk, sizeof(uint64_t) * 2 * 4 * blocks, hipMemcpyDeviceToHost));
    double cyc = 0, wall = 0;
    for (int i = 0; i < 4 * blocks; ++i) {
        cyc += (double)h[2 * i];
        wall += (double)h[2 * i + 1];
    }
    cyc /= 4 * blocks;
    wall /= 4 * blocks;
    const double mfmas = 8.0 * iters;
    const double flop = 2.0 * 32 * 32 * 16 * mfmas * 4 * blocks;
    printf("| v_mfma_f32_32x32x16_bf16, one wave per SIMD, 8 accumulators | %.2f cycles per MFMA | "
           "%.2f GHz | %.0f TFLOP/s |\n",
           cyc / mfmas, cyc / (wall / (wall_khz * 1e3)) / 1e9, flop / (ms * 1e-3) / 1e12);
    return 0;
}

// Sustained matrix rate with operands like a GEMM's: every lane holds four A and four B
// fragments of random bf16 values (random sign and mantissa, magnitudes 0.25 to 4) and
// consecutive MFMAs take different fragments, so the matrix unit's inputs toggle as they do on
// N(0,1) data. RAND = false keeps the constant near-1 operands of mfma_kernel. Launched 30 times
// back to back (a few ms each) to show the clock the package settles at.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <bool RAND>
__global__ __launch_bounds__(256) void mfma_sustained_kernel(float *out, uint64_t *clk, int iters) {
    bf16x8 a[4], b[4];
    const uint32_t lane = blockIdx.x * 256 + threadIdx.x;
    for (int f = 0; f < 4; ++f)
        for (int i = 0; i < 8; ++i) {
            const uint32_t ha = mix32(lane * 64 + f * 8 + i), hb = mix32(~(lane * 64 + f * 8 + i));
            a[f][i] = RAND ? (short)(((ha & 1u) << 15) | ((125u + ((ha >> 1) & 3u)) << 7) | ((ha >> 8) & 0x7fu))
                           : (short)(0x3f80 + (threadIdx.x & 7));
            b[f][i] = RAND ? (short)(((hb & 1u) << 15) | ((125u + ((hb >> 1) & 3u)) << 7) | ((hb >> 8) & 0x7fu))
                           : (short)(0x3c00 + i);
        }
    f32x16 acc[8];
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
    const uint64_t t1 = clock64(), w1 = wall_clock64();
    if ((threadIdx.x & 63) == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = w1 - w0;
    }
    float s = 0.0f;
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool RAND>
int run_mfma_sustained() {
    const int blocks = 256, iters = 10000, launches = 30;
    float *d;
    uint64_t *clk;
    CHECK(hipMalloc(&d, sizeof(float) * blocks * 256));
    CHECK(hipMalloc(&clk, sizeof(uint64_t) * 2 * 4 * blocks * launches));
    static uint64_t h[2 * 4 * 256 * 30];
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    hipEvent_t e[launches + 1];
    for (int i = 0; i <= launches; ++i) CHECK(hipEventCreate(&e[i]));
    CHECK(hipEventRecord(e[0]));
    for (int i = 0; i < launches; ++i) {
        hipLaunchKernelGGL(mfma_sustained_kernel<RAND>, dim3(blocks), dim3(256), 0, 0, d,
                           clk + 2 * 4 * blocks * i, iters);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e[i + 1]));
    }
    CHECK(hipEventSynchronize(e[launches]));
    CHECK(hipMemcpy(h, clk, sizeof(uint64_t) * 2 * 4 * blocks * launches, hipMemcpyDeviceToHost));
    const double flop = 2.0 * 32 * 32 * 16 * 8.0 * iters * 4 * blocks;
    for (int i = 0; i < launches; ++i) {
        if (i != 0 && i != 1 && i != 4 && i != 9 && i != 19 && i != 29) continue;
        float ms;
        CHECK(hipEventElapsedTime(&ms, e[i], e[i + 1]));
        double cyc = 0, wall = 0;
        for (int w = 0; w < 4 * blocks; ++w) {
            cyc += (double)h[2 * 4 * blocks * i + 2 * w];
            wall += (double)h[2 * 4 * blocks * i + 2 * w + 1];
        }
        printf("| %s operands | launch %d | %.3f ms | %.2f GHz | %.0f TFLOP/s |\n",
               RAND ? "random bf16" : "constant", i + 1, ms, cyc / (wall / (wall_khz * 1e3)) / 1e9,
               flop / (ms * 1e-3) / 1e12);
    }
    return 0;
}

// Sustained FP32 FMA rate at two waves per SIMD (two 256-thread workgroups per CU), 30 launches
// back to back. Registers are fixed as in valu_kernel so that no FMA pays a bank penalty:
// accumulators v32..v92 (bank 0), four src0 registers in bank 1 and four src1 registers in
// bank 3, and consecutive FMAs take different sources. RAND = false: sources 1.0 and
// accumulators 0 (little toggling); RAND = true: random sources in [-1, 1) and accumulators.
#define FMA_ROW(D0, D1, D2, D3, S1) \
    FMA1(D0, "v1", S1) FMA1(D1, "v5", S1) FMA1(D2, "v9", S1) FMA1(D3, "v13", S1)
#define FMA16_ROT                                                                          \
    FMA_ROW("v32", "v36", "v40", "v44", "v3") FMA_ROW("v48", "v52", "v56", "v60", "v7")    \
    FMA_ROW("v64", "v68", "v72", "v76", "v11") FMA_ROW("v80", "v84", "v88", "v92", "v15")
#define ROT_CLOBBERS                                                                       \
    "v1", "v3", "v5", "v7", "v9", "v11", "v13", "v15", "v32", "v36", "v40", "v44", "v48",  \
        "v52", "v56", "v60", "v64", "v68", "v72", "v76", "v80", "v84", "v88", "v92"

template <bool RAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fma_sustained_kernel(
    uint64_t *clk, int iters) {
    const uint32_t lane = blockIdx.x * 256 + threadIdx.x;
    float r[24];
    for (int i = 0; i < 24; ++i)
        r[i] = RAND ? (float)(int)(mix32(lane * 32 + i) >> 8) * (1.0f / 8388608.0f) - 1.0f
                    : (i < 8 ? 1.0f : 0.0f);
    asm volatile(
        "v_mov_b32 v1, %0\nv_mov_b32 v5, %1\nv_mov_b32 v9, %2\nv_mov_b32 v13, %3\n"
        "v_mov_b32 v3, %4\nv_mov_b32 v7, %5\nv_mov_b32 v11, %6\nv_mov_b32 v15, %7\n"
        "v_mov_b32 v32, %8\nv_mov_b32 v36, %9\nv_mov_b32 v40, %10\nv_mov_b32 v44, %11\n"
        "v_mov_b32 v48, %12\nv_mov_b32 v52, %13\nv_mov_b32 v56, %14\nv_mov_b32 v60, %15\n"
        "v_mov_b32 v64, %16\nv_mov_b32 v68, %17\nv_mov_b32 v72, %18\nv_mov_b32 v76, %19\n"
        "v_mov_b32 v80, %20\nv_mov_b32 v84, %21\nv_mov_b32 v88, %22\nv_mov_b32 v92, %23\n" ::"v"(r[0]),
        "v"(r[1]), "v"(r[2]), "v"(r[3]), "v"(r[4]), "v"(r[5]), "v"(r[6]), "v"(r[7]), "v"(r[8]), "v"(r[9]),
        "v"(r[10]), "v"(r[11]), "v"(r[12]), "v"(r[13]), "v"(r[14]), "v"(r[15]), "v"(r[16]), "v"(r[17]),
        "v"(r[18]), "v"(r[19]), "v"(r[20]), "v"(r[21]), "v"(r[22]), "v"(r[23])
        : ROT_CLOBBERS);
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) asm volatile(FMA16_ROT FMA16_ROT FMA16_ROT FMA16_ROT ::: ROT_CLOBBERS);
    const uint64_t t1 = clock64(), w1 = wall_clock64();
    if ((threadIdx.x & 63) == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = w1 - w0;
    }
}

template <bool RAND>
int run_fma_sustained() {
    const int blocks = 512, iters = 20000, launches = 30;
    uint64_t *clk;
    CHECK(hipMalloc(&clk, sizeof(uint64_t) * 2 * 4 * blocks * launches));
    static uint64_t h[2 * 4 * 512 * 30];
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    hipEvent_t e[launches + 1];
    for (int i = 0; i <= launches; ++i) CHECK(hipEventCreate(&e[i]));
    CHECK(hipEventRecord(e[0]));
    for (int i = 0; i < launches; ++i) {
        hipLaunchKernelGGL(fma_sustained_kernel<RAND>, dim3(blocks), dim3(256), 0, 0,
                           clk + 2 * 4 * blocks * i, iters);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e[i + 1]));
    }
    CHECK(hipEventSynchronize(e[launches]));
    CHECK(hipMemcpy(h, clk, sizeof(uint64_t) * 2 * 4 * blocks * launches, hipMemcpyDeviceToHost));
    const double flop = 2.0 * 64 * 64.0 * iters * 4 * blocks;
    for (int i = 0; i < launches; ++i) {
        if (i != 0 && i != 1 && i != 4 && i != 9 && i != 19 && i != 29) continue;
        float ms;
        CHECK(hipEventElapsedTime(&ms, e[i], e[i + 1]));
        double cyc = 0, wall = 0;
        for (int w = 0; w < 4 * blocks; ++w) {
            cyc += (double)h[2 * 4 * blocks * i + 2 * w];
            wall += (double)h[2 * 4 * blocks * i + 2 * w + 1];
        }
        const double ghz = cyc / (wall / (wall_khz * 1e3)) / 1e9;
        printf("| fp32 FMA, %s | launch %d | %.3f ms | %.2f GHz | %.2f cycles per FMA | %.1f TFLOP/s |\n",
               RAND ? "random operands" : "sources 1.0, accumulators from 0", i + 1, ms, ghz,
               cyc / (4.0 * blocks) / (64.0 * iters) / 2.0, flop / (ms * 1e-3) / 1e12);
    }
    return 0;
}

// ---- lds_tr: lane mapping of the transposing LDS read ---------------------------------------
// ds_read_b64_tr_b16: every lane gives an address of 4 consecutive 16-bit elements. LDS holds
// each element's own index; lane l reads row l of a 64-element-wide image (elements 64 l ..
// 64 l + 3), all in bounds of the 16 KB array. Prints which source elements each lane receives.
typedef short trv4i16 __attribute__((ext_vector_type(4)));
__global__ void lds_tr_kernel(short *out) {
    __shared__ short lds[8192];
    for (int i = threadIdx.x; i < 8192; i += 64) lds[i] = (short)i;
    __syncthreads();
    const int l = threadIdx.x;
    const trv4i16 v =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) trv4i16 *)(lds + 64 * l));
    for (int j = 0; j < 4; ++j) out[l * 4 + j] = v[j];
}

int run_lds_tr() {
    short *d;
    CHECK(hipMalloc(&d, 256 * sizeof(short)));
    hipLaunchKernelGGL(lds_tr_kernel, dim3(1), dim3(64), 0, 0, d);
    CHECK(hipGetLastError());
    static short h[256];
    CHECK(hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost));
    printf("| lane | receives (source lane . element) |\n|---|---|\n");
    for (int l = 0; l < 20; ++l) {
        printf("| %d |", l);
        for (int j = 0; j < 4; ++j) printf(" %d.%d", h[l * 4 + j] / 64, h[l * 4 + j] % 64);
        printf(" |\n");
    }
    return 0;
}

// ---- lds ----------------------------------------------------------------------------------
__device__ __forceinline__ int key_row7(int row, int c) { return row * 128 + ((c ^ (row & 7)) * 16); }
__device__ __forceinline__ int key_row7_row8(int row, int c) {
    return row * 128 + ((c ^ ((row & 7) ^ ((row >> 3) & 1))) * 16);
}

// Candidate keys for 128-byte slab rows (8 chunks of 16 bytes): chunk c of row r sits at
// c ^ key(r). Candidate 0 is the one the MFMA kernels use.
__device__ __forceinline__ int cand_key(int cand, int r) {
    const int lo = r & 7, b3 = (r >> 3) & 1;
    switch (cand) {
        case 0: return lo ^ b3;
        case 1: return lo ^ (b3 << 1);
        case 2: return lo ^ (b3 << 2);
        case 3: return lo ^ (b3 * 3);
        case 4: return ((r >> 1) & 7) ^ ((r & 1) << 2);
        default: return ((r >> 1) & 3) ^ ((r & 1) << 2) ^ (b3 << 1);
    }
}

template <int P>
__device__ __forceinline__ int lds_pattern(int lane) {
    if (P >= 100) {  // candidate key (P - 100) / 2; even P: 32x32x16 fragment read, odd: 16x16x32
        const int cand = (P - 100) / 2;
        if ((P & 1) == 0) {
            const int r = lane & 31, c = 2 + (lane >> 5);
            return r * 128 + ((c ^ cand_key(cand, r)) * 16);
        }
        const int r = lane & 15, c = 4 + (lane >> 4);
        return r * 128 + ((c ^ cand_key(cand, r)) * 16);
    }
    switch (P) {
        case 0: return lane * 16;                                 // 1 KiB contiguous
        case 1: return key_row7(lane & 31, 2 + (lane >> 5));      // 32 rows of 128 B, chunk ^ (row & 7)
        case 2: return key_row7_row8(lane & 31, 2 + (lane >> 5)); // chunk ^ ((row & 7) ^ (row >> 3 & 1))
        case 3: return (lane & 31) * 128 + (lane >> 5) * 16;      // 32 rows of 128 B, no swizzle
        case 4: return (lane >> 3) * 16;                          // 8 distinct addresses, rest broadcast
        case 5: return (lane & 1) * 256 + (lane >> 1) * 16;       // lane pairs 256 B apart
        case 7: return key_row7_row8(lane & 15, 2 + (lane >> 4)); // 16 rows x 4 chunks (16x16x32 fragment)
        case 8: return (lane & 15) * 128 + (2 + (lane >> 4)) * 16; // same, no swizzle
        default: return key_row7_row8(lane >> 3, lane & 7);       // 8 lanes per 128-byte row
    }
}

template <int P, bool WRITE>
__global__ __launch_bounds__(256) void lds_kernel(uint32_t *out, int iters) {
    __shared__ uint4 lds[4096];  // 64 KiB, 16 KiB per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4096; i += 256) lds[i] = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    int off = lds_pattern<P>(lane) + wave * 16384;  // every pattern stays below 16 KiB
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(off));
        if (WRITE) {
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(lds) + off) = make_uint4(it, it, it, it);
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(lds) + off);
            acc.x ^= v.x;
            acc.y ^= v.y;
            acc.z ^= v.z;
            acc.w ^= v.w;
        }
    }
    __syncthreads();
    out[blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w + lds[threadIdx.x].x;
}

template <int P, bool WRITE>
int lds_one(uint32_t *d, const char *what) {
    hipLaunchKernelGGL((lds_kernel<P, WRITE>), dim3(256), dim3(256), 0, 0, d, 1024);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    printf("lds pattern %d (%s) done\n", P, what);
    return 0;
}

int run_lds() {
    uint32_t *d;
    CHECK(hipMalloc(&d, sizeof(uint32_t) * 256 * 256));
    int rc = 0;
    rc |= lds_one<0, false>(d, "ds_read_b128, 1 KiB contiguous");
    rc |= lds_one<1, false>(d, "ds_read_b128, 128-byte rows, chunk ^ (row & 7)");
    rc |= lds_one<2, false>(d, "ds_read_b128, 128-byte rows, chunk ^ ((row & 7) ^ (row >> 3 & 1))");
    rc |= lds_one<3, false>(d, "ds_read_b128, 128-byte rows, no swizzle");
    rc |= lds_one<4, false>(d, "ds_read_b128, 8 distinct addresses");
    rc |= lds_one<5, false>(d, "ds_read_b128, lane pairs 256 B apart");
    rc |= lds_one<7, false>(d, "ds_read_b128, 16 rows x 4 chunks, chunk ^ ((row & 7) ^ (row >> 3 & 1))");
    rc |= lds_one<8, false>(d, "ds_read_b128, 16 rows x 4 chunks, no swizzle");
    rc |= lds_one<100, false>(d, "key candidate 0, 32x32x16 fragment");
    rc |= lds_one<101, false>(d, "key candidate 0, 16x16x32 fragment");
    rc |= lds_one<102, false>(d, "key candidate 1, 32x32x16 fragment");
    rc |= lds_one<103, false>(d, "key candidate 1, 16x16x32 fragment");
    rc |= lds_one<104, false>(d, "key candidate 2, 32x32x16 fragment");
    rc |= lds_one<105, false>(d, "key candidate 2, 16x16x32 fragment");
    rc |= lds_one<106, false>(d, "key candidate 3, 32x32x16 fragment");
    rc |= lds_one<107, false>(d, "key candidate 3, 16x16x32 fragment");
    rc |= lds_one<108, false>(d, "key candidate 4, 32x32x16 fragment");
    rc |= lds_one<109, false>(d, "key candidate 4, 16x16x32 fragment");
    rc |= lds_one<110, false>(d, "key candidate 5, 32x32x16 fragment");
    rc |= lds_one<111, false>(d, "key candidate 5, 16x16x32 fragment");
    rc |= lds_one<0, true>(d, "ds_write_b128, 1 KiB contiguous");
    rc |= lds_one<6, true>(d, "ds_write_b128, 8 lanes per 128-byte row");
    return rc;
}

int main(int argc, char **argv) {
    const char *what = argc > 1 ? argv[1] : "all";
    int rc = 0;
    if (!strcmp(what, "valu") || !strcmp(what, "all")) rc |= run_valu();
    if (!strcmp(what, "mfma") || !strcmp(what, "all")) rc |= run_mfma();
    if (!strcmp(what, "valu_sustained") || !strcmp(what, "all")) {
        rc |= run_fma_sustained<false>();
        rc |= run_fma_sustained<true>();
    }
    if (!strcmp(what, "mfma_sustained") || !strcmp(what, "all")) {
        rc |= run_mfma_sustained<false>();
        rc |= run_mfma_sustained<true>();
    }
    if (!strcmp(what, "lds")) rc |= run_lds();
    if (!strcmp(what, "lds_tr") || !strcmp(what, "all")) rc |= run_lds_tr();
    return rc;
}
