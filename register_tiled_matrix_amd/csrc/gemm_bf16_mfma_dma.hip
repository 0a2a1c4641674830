// gemm_bf16_mfma_dma.hip -- the bf16 MFMA rung for full, aligned tiles: HBM -> LDS by direct
// DMA loads, a multi-stage LDS ring, and wave tiles of 32x32x16 MFMA fragments.
//
// Same three levels as the other rungs ("寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507)
// section 1.1: global block tile -> shared tile -> register tile), with the register level
// made of MFMA fragments (section 3.2: per k step, A and B fragments are read from LDS into
// VGPRs and the C accumulators are updated in place). What is specific to gfx950 here:
//
//  * HBM -> LDS without registers: global_load_lds_dwordx4 writes each lane's 16 bytes
//    straight into LDS at (wave-uniform base + lane * 16). The LDS image of a slab is the
//    swizzled layout below, so lane l of a load instruction fetches the global chunk that
//    belongs in LDS slot (base + l): the permutation is applied to the global addresses.
//  * Slab layout: a tile row (an A row, or a B column: both operands are K-contiguous) of
//    BK bf16 is KCH = BK/8 chunks of 16 bytes; chunk c of row r sits in slot c ^ key(r).
//    128-bit LDS reads are served 16 lanes at a time over 64 banks (256 bytes). A fragment
//    read covers 16 consecutive rows at one chunk, and the key makes those 16 reads hit 16
//    distinct 16-byte bank groups:
//      KCH = 8 (128-byte rows): key(r) = (r & 7) ^ ((r >> 3) & 1)
//      KCH = 4 ( 64-byte rows): key(r) = (r >> 2) & 3
//  * STAGES slabs in flight: slab s+STAGES-1 is requested while slab s is consumed, and
//    each wave waits (s_waitcnt vmcnt) only for the slab it is about to read; one barrier
//    per slab both publishes that slab and retires the stage the next request overwrites
//    (section 6.3: prefetch of the next k-slice while the current one is computed).
//  * Wave tile WTM x WTN of 32x32 blocks: per 16-wide k step a wave reads WTM/32 A and
//    WTN/32 B fragments (one 16-byte LDS read each) and issues (WTM/32)*(WTN/32) MFMAs, so
//    LDS reads per MFMA fall as the wave tile grows.
//  * Tile order: contiguous blocks of tiles per XCD, grouped 8 tile-rows at a time.
#include "mfma_common.h"
#include "regtile_internal.h"

namespace regtile {

namespace {
using namespace mfma;

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, int MF>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void bf16_mfma_dma_kernel(
    int M, int N, int K, float alpha, const uint16_t *__restrict__ A, int64_t lda,
    const uint16_t *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int KCH = BK / 8;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    typedef Frag<MF> F;
    constexpr int MI = WTM / MF, NI = WTN / MF;
    constexpr int A_SLOTS = BM * KCH, B_SLOTS = BN * KCH;  // 16-byte slots per stage
    constexpr int STAGE_SLOTS = A_SLOTS + B_SLOTS;
    constexpr int JA = A_SLOTS / (64 * NWAVES), JB = B_SLOTS / (64 * NWAVES);
    constexpr int PER_SLAB = JA + JB;  // DMA instructions per wave per slab
    static_assert(A_SLOTS % (64 * NWAVES) == 0 && B_SLOTS % (64 * NWAVES) == 0, "even DMA split");
    static_assert(WTM % MF == 0 && WTN % MF == 0 && BK % F::KSTEP == 0, "fragment shapes");
    static_assert(PER_SLAB * (STAGES - 1) < 64, "vmcnt range");

    __shared__ uint4 smem[STAGES * STAGE_SLOTS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Global source of every slot this lane fills: slot p = (wave*J + j)*64 + lane holds
    // chunk (p % KCH) ^ key(row) of tile row p / KCH. One instruction covers 64/KCH rows, so
    // instruction j's row is instruction (j & 1)'s row plus a uniform (j & ~1) * 64/KCH, and
    // its key equals instruction (j & 1)'s (the key depends on the row only through bits that
    // an even number of instructions leaves unchanged): two per-lane pointers per operand.
    constexpr int ROWS_PER_INSTR = 64 / KCH;
    static_assert(KCH == 4 || (ROWS_PER_INSTR == 8 && JA % 2 == 0 && JB % 2 == 0), "key periodicity");
    const uint16_t *a_lane[2];
    const uint16_t *b_lane[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int pa = (wave * JA + j) * 64 + lane;
        const int ra = pa / KCH, ca = (pa % KCH) ^ slab_key<KCH>(ra);
        a_lane[j] = A + (int64_t)(m0 + ra) * lda + ca * 8;
        const int pb = (wave * JB + j) * 64 + lane;
        const int rb = pb / KCH, cb = (pb % KCH) ^ slab_key<KCH>(rb);
        b_lane[j] = B + (int64_t)(n0 + rb) * ldb + cb * 8;
    }
    const int64_t a_step = (int64_t)ROWS_PER_INSTR * lda;  // per instruction pair: 2 * a_step
    const int64_t b_step = (int64_t)ROWS_PER_INSTR * ldb;
    auto a_src = [&](int j) { return a_lane[j & 1] + (j & ~1) * a_step; };
    auto b_src = [&](int j) { return b_lane[j & 1] + (j & ~1) * b_step; };

    auto issue = [&](int slab, int stage) {
        const int k0 = slab * BK;
        uint4 *sa = smem + stage * STAGE_SLOTS;
        uint4 *sb = sa + A_SLOTS;
#pragma unroll
        for (int j = 0; j < JA; ++j)
            dma16(a_src(j) + k0, sa + (wave * JA + j) * 64);
#pragma unroll
        for (int j = 0; j < JB; ++j)
            dma16(b_src(j) + k0, sb + (wave * JB + j) * 64);
    };

    typename F::acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < F::NACC; ++v) acc[i][j][v] = 0.0f;

    const int frag_r = lane % MF;   // fragment row (A) / column (B) of this lane
    const int frag_kg = lane / MF;  // its group of 8 k values within the instruction's k step

    // Fragment reads of one k step (F::KSTEP wide) into register buffer `buf`. Every group
    // of MF lanes reads MF consecutive slab rows at one chunk: conflict-free under the key.
    bf16x8 fa[2][MI], fb[2][NI];
    auto read_frags = [&](const uint4 *sa, const uint4 *sb, int kk, int buf) {
        const int chunk = kk * (F::KSTEP / 8) + frag_kg;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int row = wm * WTM + i * MF + frag_r;
            fa[buf][i] = __builtin_bit_cast(bf16x8, sa[row * KCH + (chunk ^ slab_key<KCH>(row))]);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int row = wn * WTN + j * MF + frag_r;
            fb[buf][j] = __builtin_bit_cast(bf16x8, sb[row * KCH + (chunk ^ slab_key<KCH>(row))]);
        }
    };
    // One slab. Each 16-wide k step starts by waiting for its own fragments (read during the
    // previous step), then issues its MFMAs with the next step's fragment reads and a share
    // of the next slab's DMA loads woven between them: MFMA, read, MFMA, DMA, ... A 1 KB DMA
    // instruction occupies the wave's issue for about 20 cycles (the address unit moves
    // 64 bytes per clock), less than one 32-cycle MFMA, so spread out it costs no matrix
    // cycles, while a burst of them would stall the MFMAs queued behind it.
    constexpr int KSTEPS = BK / F::KSTEP;
    constexpr int NMFMA = MI * NI;
    constexpr int NREAD = MI + NI;
    constexpr int DMA_PER_STEP = (PER_SLAB + KSTEPS - 1) / KSTEPS;
    static_assert(NREAD <= NMFMA && DMA_PER_STEP <= NMFMA, "one extra instruction per MFMA slot");
    auto compute = [&](int stage, int next_slab, int next_stage) {
        const uint4 *sa = smem + stage * STAGE_SLOTS;
        const uint4 *sb = sa + A_SLOTS;
        const int k0n = next_slab * BK;
        uint4 *na = smem + next_stage * STAGE_SLOTS;
        uint4 *nb = na + A_SLOTS;
        read_frags(sa, sb, 0, 0);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int cb = kk & 1;
            wait_lgkmcnt0();  // this step's fragments have landed
            __builtin_amdgcn_sched_barrier(0);
            if (kk + 1 < KSTEPS) read_frags(sa, sb, kk + 1, cb ^ 1);
#pragma unroll
            for (int d = 0; d < DMA_PER_STEP; ++d) {
                const int q = kk * DMA_PER_STEP + d;  // DMA instruction index within the slab
                if (q < JA) dma16(a_src(q) + k0n, na + (wave * JA + q) * 64);
                else if (q < PER_SLAB) dma16(b_src(q - JA) + k0n, nb + (wave * JB + (q - JA)) * 64);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = F::mfma(fa[cb][i], fb[cb][j], acc[i][j]);
            // issue order: every MFMA is followed by at most one read or one DMA
            const int reads = (kk + 1 < KSTEPS) ? NREAD : 0;
            const int dmas = (kk * DMA_PER_STEP < PER_SLAB)
                                     ? ((PER_SLAB - kk * DMA_PER_STEP) < DMA_PER_STEP
                                            ? (PER_SLAB - kk * DMA_PER_STEP) : DMA_PER_STEP)
                                     : 0;
            int r_left = reads, d_left = dmas;
#pragma unroll
            for (int g = 0; g < NMFMA; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                // spread reads and DMAs evenly over the MFMA slots
                const bool want_dma = d_left > 0 && (g * dmas) / NMFMA != ((g + 1) * dmas) / NMFMA;
                if (want_dma) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    --d_left;
                } else if (r_left > 0) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    --r_left;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Every iteration requests exactly one slab, so the wait count is the same each time.
    // Past the end the request is clamped to the last slab: it rewrites a stage that has
    // already been consumed with valid data and keeps the loop body uniform.
    const int nslabs = K / BK;
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) issue(min(t, nslabs - 1), t);

    for (int s = 0; s < nslabs; ++s) {
        // Slab s must have landed; the requests of the STAGES-2 slabs after it may still fly.
        wait_vmcnt<PER_SLAB * (STAGES - 2)>();
        __syncthreads();
        const int next = s + STAGES - 1;
        compute(s % STAGES, min(next, nslabs - 1), next % STAGES);
    }
    wait_vmcnt<0>();  // no LDS DMA may still be in flight when the workgroup retires

    // Epilogue: accumulator v of a fragment lands at (row_lane + row_acc(v), lane % MF) of
    // its MF x MF block. beta == 0 never reads C.
    const bool read_c = beta != 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = n0 + wn * WTN + j * MF + frag_r;
            float *cbase = C + (int64_t)(m0 + wm * WTM + i * MF + F::row_lane(lane)) * ldc + col;
            if (read_c) {
#pragma unroll
                for (int v = 0; v < F::NACC; ++v) {
                    float *c = cbase + (int64_t)F::row_acc(v) * ldc;
                    *c = fmaf(alpha, acc[i][j][v], beta * *c);
                }
            } else {
#pragma unroll
                for (int v = 0; v < F::NACC; ++v)
                    cbase[(int64_t)F::row_acc(v) * ldc] = alpha * acc[i][j][v];
            }
        }
    }
}

template <int BM, int BN, int BK, int STAGES, int WM, int WN, int MF>
hipError_t launch_dma_cfg(const Problem &p, hipStream_t s) {
    const int tiles_m = p.M / BM, tiles_n = p.N / BN;
    hipLaunchKernelGGL((bf16_mfma_dma_kernel<BM, BN, BK, STAGES, WM, WN, MF>), dim3(tiles_m * tiles_n),
                       dim3(WM * WN * 64), 0, s, p.M, p.N, p.K, p.alpha, (const uint16_t *)p.A,
                       p.lda, (const uint16_t *)p.B, p.ldb, p.beta, p.C, p.ldc, tiles_m, tiles_n);
    return hipGetLastError();
}



#ifndef DMA_BM
#define DMA_BM 256
#define DMA_BN 256
#define DMA_BK 64
#define DMA_STAGES 2
#define DMA_WM 2
#define DMA_WN 2
#endif

}  // namespace

// Returns hipErrorNotSupported (and launches nothing) unless the problem is made of full
// tiles with 16-byte aligned, K-contiguous rows.
hipError_t launch_bf16_mfma_dma(const Problem &p, hipStream_t s, const char **name, int shape) {
    const bool ok = p.M % DMA_BM == 0 && p.N % DMA_BN == 0 && p.K % DMA_BK == 0 && p.K > 0 &&
                    p.lda % 8 == 0 && p.ldb % 8 == 0 && aligned16(p.A) && aligned16(p.B) &&
                    (int64_t)(p.M / DMA_BM) * (p.N / DMA_BN) >= 128 && (shape == 32 || shape == 16);
    if (!ok) return hipErrorNotSupported;
#define REGTILE_DMA_NAME(mf)                                                                   \
    "bf16_mfma" mf "_dma_" REGTILE_STR(DMA_BM) "x" REGTILE_STR(DMA_BN) "x" REGTILE_STR(DMA_BK) \
        "_s" REGTILE_STR(DMA_STAGES) "_w" REGTILE_STR(DMA_WM) "x" REGTILE_STR(DMA_WN)
    if (shape == 16) {
        *name = REGTILE_DMA_NAME("16x16x32");
        return launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_STAGES, DMA_WM, DMA_WN, 16>(p, s);
    }
    *name = REGTILE_DMA_NAME("32x32x16");
    return launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_STAGES, DMA_WM, DMA_WN, 32>(p, s);
#undef REGTILE_DMA_NAME
}

}  // namespace regtile
