// gemm_bf16_mfma_dma.hip -- the bf16 / fp16 MFMA kernel: HBM -> LDS by direct DMA loads
// through per-tile buffer descriptors, a multi-stage LDS ring, and wave tiles of MFMA
// fragments. It takes every problem whose rows are 16-byte aligned (M, N and K may end inside
// a tile); others go to the register-staged kernel (gemm_bf16_mfma.hip).
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
//    The key is chosen per fragment shape by measurement (LDS bank-conflict counters on the
//    fragment read patterns; mfma_common.h) so that the fragment reads are conflict-free:
//      KCH = 8, MF = 32: key(r) = (r & 7) ^ ((r >> 3) & 1)
//      KCH = 8, MF = 16: key(r) = ((r >> 1) & 7) ^ ((r & 1) << 2)
//      KCH = 4 (64-byte rows): key(r) = (r >> 2) & 3
//  * M/N-contiguous operands: as rows staged through registers ("n n", "t t"), or in their own
//    storage with transposing fragment reads ("t n"); see the kernel.
//  * Edges: every descriptor ends at the last element of the matrix it covers
//    (tile_addressing.h), so loads past it read zeros and stores past it are dropped; columns
//    past N get an out-of-range store offset; chunks past K in the last slab an out-of-range
//    load offset. Nothing outside the caller's matrices is read or written.
//  * Two LDS stages and one barrier per slab, placed inside the slab's last k step: the
//    next slab is loaded while the current one is consumed, and its first fragments are
//    read before the current slab's last MFMAs (section 6.3: prefetch of the next k slice
//    while the current one is computed). The barrier carries no memory fence; each wave
//    waits (s_waitcnt vmcnt) for exactly its own loads before it.
//  * Wave tile WTM x WTN of 32x32 blocks: per 16-wide k step a wave reads WTM/32 A and
//    WTN/32 B fragments (one 16-byte LDS read each) and issues (WTM/32)*(WTN/32) MFMAs, so
//    LDS reads per MFMA fall as the wave tile grows.
//  * Tile order: contiguous blocks of tiles per XCD, grouped 8 tile-rows at a time.
#include <type_traits>

#include "mfma_common.h"
#include "regtile_internal.h"

// 1: each k step's MFMAs walk the wave tile's fragment grid row by row in alternating
// column order, so consecutive MFMAs always share one operand (fewer operand bits switch from
// one MFMA to the next; the package's clock on random data is power-bound); 0: row by row,
// left to right. Either order gives every accumulator the same sequence of k steps.
#ifndef DMA_SNAKE
#define DMA_SNAKE 1
#endif

namespace regtile {

namespace {
using namespace mfma;

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MF, int WINDOWS, int STAGGER, bool F16,
          int RING = 2, int ROWS = 0, bool KTAIL = false, int MN = 0>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void bf16_mfma_dma_kernel(
    int M, int N, int K, float alpha, const uint16_t *__restrict__ A, int64_t lda,
    const uint16_t *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int KCH = BK / 8;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    typedef Frag<MF, F16> F;
    constexpr int MI = WTM / MF, NI = WTN / MF;
    constexpr int A_SLOTS = BM * KCH, B_SLOTS = BN * KCH;  // 16-byte slots per stage
    constexpr int STAGE_SLOTS = A_SLOTS + B_SLOTS;
    constexpr int JA = A_SLOTS / (64 * NWAVES), JB = B_SLOTS / (64 * NWAVES);
    constexpr int PER_SLAB = JA + JB;  // DMA instructions per wave per slab
    static_assert(A_SLOTS % (64 * NWAVES) == 0 && B_SLOTS % (64 * NWAVES) == 0, "even DMA split");
    static_assert(WTM % MF == 0 && WTN % MF == 0 && BK % F::KSTEP == 0, "fragment shapes");
    static_assert(PER_SLAB < 64, "vmcnt range");
    constexpr int STAGES = 2;
    static_assert(RING == 2 || (RING == 5 && A_SLOTS == B_SLOTS), "two stages, or a ring of five halves");
    // ROWS: 0 both operands K-contiguous over DMA; 1 B stored K x N (N-contiguous); 2 A stored
    // K x M (M-contiguous). The M/N-contiguous operand arrives as rows through registers.
    constexpr bool A_ROW = ROWS == 2, ANY_ROW = ROWS != 0;
    static_assert(ROWS >= 0 && ROWS <= 2 && (!ANY_ROW || RING == 5), "row operands go through the ring");
    // KTAIL: K ends inside the last slab (K a multiple of 8, so each 16-byte chunk lies wholly
    // before or wholly past K); that slab's chunks past K are loaded from an offset past the
    // descriptor's end, which puts zeros in LDS.
    // MN: bit 0, A is stored K x M; bit 1, B is stored K x N. Such an operand keeps its storage
    // in LDS: a slab of BK rows (k) of BM (BN) elements, 16-byte chunk c of row r at slot
    // c ^ mn_key(r). Its DMA reads through a descriptor over its K rows from the tile's first
    // column that ends at the operand's last element (rows past K read zeros; other columns
    // past M or N only feed dropped outputs), and its fragments come from pairs of
    // transposing LDS reads.
    constexpr bool A_MN = (MN & 1) != 0, B_MN = (MN & 2) != 0;
    static_assert(MN == 0 || (ROWS == 0 && RING == 5 && MF == 32 && BM == BN && (BM == 256 || BM == 128) && BK == 64),
                  "M/N-major slabs: 32x32x16 fragments on the 256x256 or 128x128 ring");


    __shared__ uint4 smem[RING == 5 ? 5 * A_SLOTS : STAGES * STAGE_SLOTS];

    const int tid = threadIdx.x;
    // wave-uniform by construction; readfirstlane tells the compiler so (scalar registers
    // for everything derived from it, and a scalar M0 for the LDS DMA destination)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Global source of every slot this lane fills: slot p = (wave*J + j)*64 + lane holds
    // chunk (p % KCH) ^ key(row) of tile row p / KCH. One instruction covers 64/KCH rows, so
    // instruction j's row is instruction (j & 1)'s row plus a uniform (j & ~1) * 64/KCH, and
    // its key equals instruction (j & 1)'s (the key depends on the row only through bits that
    // an even number of instructions leaves unchanged). Loads go through buffer descriptors
    // over the tile's BM rows of A and BN rows of B: per lane two 32-bit byte offsets per
    // operand; instruction and slab offsets are wave-uniform (SGPR).
    constexpr int ROWS_PER_INSTR = 64 / KCH;
    static_assert(KCH == 4 || (ROWS_PER_INSTR == 8 && JA % 2 == 0 && JB % 2 == 0), "key periodicity");
    // Every descriptor ends at the last element of the matrix it reads (tile_addressing.h):
    // a K-contiguous tile's at element K - 1 of its last real row, so that DMA loads of rows
    // past M (N) read zeros; an M/N-major operand's at column M - 1 (N - 1) of row K - 1, so
    // that rows past K and that row's columns past M (N) read zeros. The launchers admit an
    // M/N-major operand only when its column count and leading dimension are multiples of 8,
    // so no 16-byte chunk straddles that end.
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const rsrc_t a_rsrc = A_MN ? make_rsrc(A + m0, addr::desc_bytes(K, lda, M - m0, 2))
                               : make_rsrc(A + (int64_t)m0 * lda, addr::desc_bytes(rows_a, lda, K, 2));
    const rsrc_t b_rsrc = B_MN ? make_rsrc(B + n0, addr::desc_bytes(K, ldb, N - n0, 2))
                               : make_rsrc(B + (int64_t)n0 * ldb, addr::desc_bytes(rows_b, ldb, K, 2));
    const int nslabs = KTAIL ? (K + BK - 1) / BK : K / BK;
    const int k_last = (nslabs - 1) * BK;  // first k of the last slab
    // An M/N-major slab row holds MCH chunks; one DMA instruction covers MROWS = 64 / MCH rows.
    constexpr int MCH = BM / 8, MROWS = 64 / MCH;
    uint32_t a_voff[2], b_voff[2], a_voff_last[2], b_voff_last[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int ka, kb;  // first k of each lane's chunk within the slab
        a_voff[j] = addr::kc_dma_lane<KCH, MF>(wave, JA, j, lane, lda, &ka);
        b_voff[j] = addr::kc_dma_lane<KCH, MF>(wave, JB, j, lane, ldb, &kb);
        // (the uniform parts added to kPastEnd stay below 2^32)
        a_voff_last[j] = k_last + ka < K ? a_voff[j] : a_voff[j] | addr::kPastEnd;
        b_voff_last[j] = k_last + kb < K ? b_voff[j] : b_voff[j] | addr::kPastEnd;
        if (A_MN) a_voff[j] = addr::mn_dma_lane(lane, j, lda, MCH);
        if (B_MN) b_voff[j] = addr::mn_dma_lane(lane, j, ldb, MCH);
    }
    static_assert(MN == 0 || (JA % 2 == 0 && JB % 2 == 0 && (MROWS == 2 || MROWS == 4)),
                  "two or four rows per instruction");
    auto voff_a = [&](int q, int k0) {
        return KTAIL && !A_MN && k0 == k_last ? a_voff_last[q & 1] : a_voff[q & 1];
    };
    auto voff_b = [&](int q, int k0) {
        return KTAIL && !B_MN && k0 == k_last ? b_voff_last[q & 1] : b_voff[q & 1];
    };
    // uniform byte offset of DMA instruction q of the slab starting at k0
    auto soff_a = [&](int q, int k0) {
        return A_MN ? addr::mn_dma_instr(wave, JA, q, k0, lda, MCH) : addr::kc_dma_instr<KCH>(q, k0, lda);
    };
    auto soff_b = [&](int q, int k0) {
        return B_MN ? addr::mn_dma_instr(wave, JB, q, k0, ldb, MCH) : addr::kc_dma_instr<KCH>(q, k0, ldb);
    };
    // DMA instruction q (A for q < JA, then B) of the slab starting at k0.
    auto dma_q = [&](int q, int k0, uint4 *sa, uint4 *sb) {
        if (q < JA)
            dma16_buf(a_rsrc, voff_a(q, k0), soff_a(q, k0), sa + (wave * JA + q) * 64);
        else
            dma16_buf(b_rsrc, voff_b(q - JA, k0), soff_b(q - JA, k0), sb + (wave * JB + (q - JA)) * 64);
    };

    // One DMA instruction q of the A part (B part) of the slab starting at k0 into the half
    // (A or B area) at `dst`.
    auto dma_a = [&](int q, int k0, uint4 *dst) {
        dma16_buf(a_rsrc, voff_a(q, k0), soff_a(q, k0), dst + (wave * JA + q) * 64);
    };
    auto dma_b = [&](int q, int k0, uint4 *dst) {
        dma16_buf(b_rsrc, voff_b(q, k0), soff_b(q, k0), dst + (wave * JB + q) * 64);
    };
    // the operand that keeps its DMA when the other arrives as rows
    auto dma_e = [&](int q, int k0, uint4 *dst) {
        if constexpr (A_ROW)
            dma_b(q, k0, dst);
        else
            dma_a(q, k0, dst);
    };

    // The row operand (ANY_ROW) has no DMA. Each thread owns 4 x 8 blocks of its slab (4
    // consecutive m or n, 8 consecutive k; two blocks on 256x256 tiles, one on 128x128), reads
    // them as 8-byte runs along m or n (consecutive lanes take consecutive runs of one k row),
    // and after the half they go to is free writes them transposed (8 k per 16-byte chunk,
    // mfma_common.h) into the swizzled slab.
    constexpr int NT = NWAVES * 64;
    constexpr int RLEN = A_ROW ? BM : BN;  // slab rows of the row operand
    constexpr int B_BLOCKS = ANY_ROW ? (RLEN / 4) * KCH / NT : 1;
    static_assert(!ANY_ROW || (B_BLOCKS >= 1 && (RLEN / 4) * KCH == B_BLOCKS * NT),
                  "whole 4 x 8 blocks per thread");
    constexpr int NBL = ANY_ROW ? B_BLOCKS * 8 : 0;  // row loads per thread per slab
    // The row operand's loads go through a descriptor over its K rows (of ld_row elements)
    // from the tile's first column, ending at its last element: rows at or past K read zeros
    // (the K tail), and so do the last row's columns past M or N (the launcher admits a row
    // operand only when its column count and leading dimension are multiples of 4, so no
    // 8-byte run straddles that end). Other columns past M or N read the operand's own
    // storage and only feed outputs that are never stored.
    const uint16_t *const rsrc_base = A_ROW ? A + m0 : B + n0;
    const int64_t ld_row = A_ROW ? lda : ldb;
    const rsrc_t row_rsrc = make_rsrc(rsrc_base, addr::desc_bytes(K, ld_row, A_ROW ? M - m0 : N - n0, 2));
    uint32_t bl[B_BLOCKS][8], bh[B_BLOCKS][8];
    int brow_n[B_BLOCKS], brow_kc[B_BLOCKS];
    uint32_t brow_off[B_BLOCKS];
#pragma unroll
    for (int i = 0; i < B_BLOCKS; ++i) {
        const int b = tid + NT * i;
        brow_n[i] = addr::row_block_col(b, RLEN);
        brow_kc[i] = addr::row_block_kc(b, RLEN);
        brow_off[i] = addr::row_block_off(b, RLEN, ld_row);
    }
    auto load_brow = [&](int slab) {
        const int k0 = min(slab, nslabs - 1) * BK;
#pragma unroll
        for (int i = 0; i < B_BLOCKS; ++i)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const uint2 v = load_b64_buf(row_rsrc, brow_off[i], addr::row_run_off(k0 + kk, ld_row));
                bl[i][kk] = v.x;
                bh[i][kk] = v.y;
            }
    };
    auto write_brow = [&](uint4 *dst) {
#pragma unroll
        for (int i = 0; i < B_BLOCKS; ++i) {
            uint4 out[4];
            transpose_4x8(bl[i], bh[i], out);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = brow_n[i] + j;
                dst[row * KCH + (brow_kc[i] ^ slab_key<KCH, MF>(row))] = out[j];
            }
        }
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
    // M/N-major fragment: lane l needs column c of the fragment (c = l % 32) at k = 8 (l / 32)
    // .. +7 of the k step. In each group of 16 lanes, lane t addresses row k + t / 4 (+ 4 for
    // the second read) at columns 16 ((l / 16) % 2) + 4 (t % 4) .. +3, so that lane t receives
    // column 16 ((l / 16) % 2) + t of four consecutive rows (the transposing read's mapping).
    const int tr_t = lane & 15;
    const int tr_row = 8 * (lane >> 5) + (tr_t >> 2);                    // row within the k step
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_t & 3);         // column within the fragment
    auto mn_frag = [&](const uint4 *slab, int col0, int kk) {
        const char *base = reinterpret_cast<const char *>(slab);
        const int row = kk * F::KSTEP + tr_row, col = col0 + tr_col;
        // row & 3 == tr_t >> 2 for both reads (rows 4 apart)
        const int off = ((col >> 3) ^ addr::mn_key(row)) * 16 + (col & 7) * 2;
        const uint2 lo = lds_read_tr16(base + row * (MCH * 16) + off);
        const uint2 hi = lds_read_tr16(base + (row + 4) * (MCH * 16) + off);
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    auto read_frags = [&](const uint4 *sa, const uint4 *sb, int kk, int buf) {
        const int chunk = kk * (F::KSTEP / 8) + frag_kg;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if constexpr (A_MN) {
                fa[buf][i] = mn_frag(sa, wm * WTM + i * MF, kk);
            } else {
                const int row = wm * WTM + i * MF + frag_r;
                fa[buf][i] = __builtin_bit_cast(bf16x8, sa[row * KCH + (chunk ^ slab_key<KCH, MF>(row))]);
            }
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if constexpr (B_MN) {
                fb[buf][j] = mn_frag(sb, wn * WTN + j * MF, kk);
            } else {
                const int row = wn * WTN + j * MF + frag_r;
                fb[buf][j] = __builtin_bit_cast(bf16x8, sb[row * KCH + (chunk ^ slab_key<KCH, MF>(row))]);
            }
        }
    };
    // One slab is KSTEPS k steps. Each starts by waiting for its own fragments (read during
    // the previous step) and issues its MFMAs with the next step's fragment reads and a
    // window of DMA loads woven between them: MFMA, read, MFMA, DMA, ... so the matrix pipe
    // never waits on an LDS round trip, and DMA issue (which can hold the wave while the
    // CU's address unit is busy) is spread thin.
    //
    // Two LDS stages, cur = s % 2 and nxt. The single barrier of a slab sits at the start
    // of its last k step, when every wave has its last fragments of stage cur in registers
    // and has waited for its own loads of slab s+1. After it, stage nxt is published and
    // stage cur is free, so the same k step already reads slab s+1's first fragments and
    // starts loading slab s+2 into stage cur. The DMA of a slab goes out in NWIN windows:
    // right after that barrier, then in the first NWIN-1 k steps of the next slab, so every
    // load has more than a k step to land before the barrier that waits for it.
    constexpr int KSTEPS = BK / F::KSTEP;
    constexpr int NMFMA = MI * NI;
    constexpr int NREAD = MI * (A_MN ? 2 : 1) + NI * (B_MN ? 2 : 1);  // LDS reads per k step
    constexpr int NWIN = KSTEPS - 1 < WINDOWS ? KSTEPS - 1 : WINDOWS;
    constexpr int JE = A_ROW ? JB : JA;  // DMA instructions of the early (DMA) operand
    constexpr int PER_SET = ANY_ROW ? JE : PER_SLAB;  // DMA instructions per wave and slab
    constexpr int DMA_PER_WIN = (PER_SET + NWIN - 1) / NWIN;
    static_assert(KSTEPS % 2 == 0 && NWIN >= 1, "even number of k steps per slab");
    // (transposing reads on 64x64 wave tiles: 8 per k step against 4 MFMAs, two per slot)
    static_assert((NREAD <= NMFMA || (MN != 0 && NREAD <= 2 * NMFMA)) && DMA_PER_WIN <= NMFMA,
                  "one extra instruction per MFMA slot, or two fragment reads");

    auto dma_window = [&](int slab, int stage, int win) {
        const int k0 = slab * BK;
        uint4 *sa = smem + stage * STAGE_SLOTS;
        uint4 *sb = sa + A_SLOTS;
#pragma unroll
        for (int d = 0; d < DMA_PER_WIN; ++d) {
            const int q = win * DMA_PER_WIN + d;  // DMA instruction index within the slab
            if (q < PER_SLAB) dma_q(q, k0, sa, sb);
        }
    };
    auto dmas_in = [](int win) {
        const int left = PER_SET - win * DMA_PER_WIN;
        return left <= 0 ? 0 : (left < DMA_PER_WIN ? left : DMA_PER_WIN);
    };
    // MFMAs of buffer cb; every MFMA is followed by at most one fragment read or one DMA.
    auto mfma_woven = [&](int cb, int reads, int dmas) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                const int j = (DMA_SNAKE && (i & 1)) ? NI - 1 - jj : jj;
                acc[i][j] = F::mfma(fa[cb][i], fb[cb][j], acc[i][j]);
            }
        int r_left = reads, d_left = dmas;
#pragma unroll
        for (int g = 0; g < NMFMA; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            const bool want_dma = d_left > 0 && (g * dmas) / NMFMA != ((g + 1) * dmas) / NMFMA;
            if (want_dma) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                --d_left;
            } else if (r_left > 0) {
                if (NREAD > NMFMA && r_left > 1) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    r_left -= 2;
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    --r_left;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // The same MFMAs with several kinds of other instructions spread evenly over the MFMA
    // slots: vector-memory loads, LDS reads, VALU (the B transposes) and LDS writes (at most
    // 2, 2, 4 and 2 per slot).
    auto mfma_spread = [&](int cb, int reads, int vmem, int valu, int dsw) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                const int j = (DMA_SNAKE && (i & 1)) ? NI - 1 - jj : jj;
                acc[i][j] = F::mfma(fa[cb][i], fb[cb][j], acc[i][j]);
            }
#pragma unroll
        for (int g = 0; g < NMFMA; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            const int nv = ((g + 1) * vmem) / NMFMA - (g * vmem) / NMFMA;
            const int nr = ((g + 1) * reads) / NMFMA - (g * reads) / NMFMA;
            const int na = ((g + 1) * valu) / NMFMA - (g * valu) / NMFMA;
            const int nw = ((g + 1) * dsw) / NMFMA - (g * dsw) / NMFMA;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (t < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (t < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t < na) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (t < nw) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Past the end, requests are clamped to the last slab: they refill a stage nobody reads
    // again with valid data and keep every iteration identical (same counts at every wait).
    if constexpr (RING == 2) {
#pragma unroll
        for (int q = 0; q < PER_SLAB; ++q) dma_q(q, 0, smem, smem + A_SLOTS);
        wait_vmcnt<0>();
        lds_barrier();
        read_frags(smem, smem + A_SLOTS, 0, 0);
    }

    // DMA windows sit at positions of the k-step sequence: position 0 is the last k step of
    // a slab (after its barrier), position p >= 1 is k step p-1 of the next slab. Window w of
    // a wave with shift SH sits at position SH + w. With STAGGER the second half of the
    // waves is shifted by one position, so on each SIMD (waves w and w + 4 of eight share
    // one) only one wave issues DMA in a given k step while the other keeps the matrix pipe
    // busy, and the CU's address unit sees half the burst.
    auto main_loop = [&](auto shift_tag) {
        constexpr int SH = decltype(shift_tag)::value;
        static_assert(SH + NWIN <= KSTEPS, "every window lands at least one k step before its barrier");
        if (SH == 0) dma_window(min(1, nslabs - 1), 1, 0);
        for (int s = 0; s < nslabs; ++s) {
            const int cur = s & 1, nxt = cur ^ 1;
            const uint4 *sa = smem + cur * STAGE_SLOTS, *sb = sa + A_SLOTS;
            const uint4 *na = smem + nxt * STAGE_SLOTS, *nb = na + A_SLOTS;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int cb = kk & 1;
                wait_lgkmcnt0();  // this step's fragments have landed
                if (kk + 1 < KSTEPS) {
                    __builtin_amdgcn_sched_barrier(0);
                    read_frags(sa, sb, kk + 1, cb ^ 1);
                    const int win = kk + 1 - SH;
                    const bool has = win >= 0 && win < NWIN;
                    if (has) dma_window(min(s + 1, nslabs - 1), nxt, win);
                    mfma_woven(cb, NREAD, has ? dmas_in(win) : 0);
                } else {
                    wait_vmcnt<0>();  // own loads of slab s+1 have landed
                    lds_barrier();    // slab s+1 published; stage cur read by nobody any more
                    read_frags(na, nb, 0, cb ^ 1);
                    if (SH == 0) dma_window(min(s + 2, nslabs - 1), cur, 0);
                    mfma_woven(cb, NREAD, SH == 0 ? dmas_in(0) : 0);
                }
            }
        }
    };
    // Ring of five half-stages (RING == 5): all of LDS as five 32 KB halves, slab t's A part
    // in half (2t) % 5 and its B part in half (2t + 1) % 5. While slab s is consumed, slab
    // s+1 is in two more halves and slab s+2's A part in the fifth, so after the barrier that
    // frees slab s's two halves a wave loads B of slab s+2 and A of slab s+3 into them. A
    // parts thus get about two slabs to land, and the barrier before slab s+1's last k step
    // waits only for B of slab s+2 (the A loads issued after it may stay in flight).
    auto ring_window = [&](int win, int slab_b, int h_b, int slab_a, int h_a) {
        const int kb = min(slab_b, nslabs - 1) * BK, ka = min(slab_a, nslabs - 1) * BK;
#pragma unroll
        for (int d = 0; d < DMA_PER_WIN; ++d) {
            const int q = win * DMA_PER_WIN + d;  // B instructions first, then A
            if constexpr (ANY_ROW) {  // only the DMA operand; the other arrives as rows
                if (q < JE) dma_e(q, ka, smem + h_a * A_SLOTS);
            } else if (q < JB) {
                dma_b(q, kb, smem + h_b * A_SLOTS);
            } else if (q < PER_SLAB) {
                dma_a(q - JB, ka, smem + h_a * A_SLOTS);
            }
        }
    };
    auto wrap5 = [](int h) { return h >= 5 ? h - 5 : h; };
    auto ring_loop = [&](auto shift_tag) {
        constexpr int SH = decltype(shift_tag)::value;
        static_assert(SH + NWIN <= KSTEPS, "every window lands at least one k step before its barrier");
        // prologue: A and B of slab 0, A of slab 1, and (unshifted waves) the first window of
        // the set a barrier before slab 0 would have issued: B of slab 1, A of slab 2
#pragma unroll
        for (int q = 0; q < JA; ++q) dma_a(q, 0, smem);
#pragma unroll
        for (int q = 0; q < JB; ++q) dma_b(q, 0, smem + A_SLOTS);
#pragma unroll
        for (int q = 0; q < JA; ++q) dma_a(q, min(1, nslabs - 1) * BK, smem + 2 * A_SLOTS);
        if (SH == 0) ring_window(0, 1, 3, 2, 4);
        wait_vmcnt<JA + (SH == 0 ? dmas_in(0) : 0)>();  // A and B of slab 0 have landed
        lds_barrier();
        read_frags(smem, smem + A_SLOTS, 0, 0);
        int ha = 0;  // half of slab s's A part; its B part is in ha + 1
        for (int s = 0; s < nslabs; ++s) {
            const int hb = wrap5(ha + 1), hna = wrap5(ha + 2), hnb = wrap5(ha + 3), hfa = wrap5(ha + 4);
            const uint4 *sa = smem + ha * A_SLOTS, *sb = smem + hb * A_SLOTS;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int cb = kk & 1;
                wait_lgkmcnt0();
                if (kk + 1 < KSTEPS) {
                    __builtin_amdgcn_sched_barrier(0);
                    read_frags(sa, sb, kk + 1, cb ^ 1);
                    // windows of the set issued after the previous slab's barrier:
                    // B of slab s+1 (half hnb) and A of slab s+2 (half hfa)
                    const int win = kk + 1 - SH;
                    const bool has = win >= 0 && win < NWIN;
                    if (has) ring_window(win, s + 1, hnb, s + 2, hfa);
                    mfma_woven(cb, NREAD, has ? dmas_in(win) : 0);
                } else {
                    wait_vmcnt<JA>();  // B of slab s+1 landed (A of slab s+2 may be in flight)
                    lds_barrier();     // slab s+1 published; slab s's halves read by nobody
                    read_frags(smem + hna * A_SLOTS, smem + hnb * A_SLOTS, 0, cb ^ 1);
                    if (SH == 0) ring_window(0, s + 2, ha, s + 3, hb);
                    mfma_woven(cb, NREAD, SH == 0 ? dmas_in(0) : 0);
                }
            }
            ha = wrap5(ha + 2);
        }
    };
    // Ring with a row operand (ANY_ROW): the DMA operand takes the early half of each slab
    // ((2t) % 5), the row operand the late one ((2t + 1) % 5). In k step 2 of slab s a wave
    // writes the rows of slab s+1 (read into registers one slab earlier), transposed, into
    // their half (freed by slab s-1's barrier), then reads slab s+2's rows into the same
    // registers: four k steps to land. The vector-memory order per wave is ... rows (s+1),
    // DMA (s+2), rows (s+2), DMA (s+3) ..., so waiting for the rows of slab s+1 leaves JE
    // operations in flight, and the barrier needs no vector-memory wait at all (the DMA of slab
    // s+1 precedes those rows).
    auto frags_at = [&](int h_early, int h_late, int kk, int buf) {
        if constexpr (A_ROW)
            read_frags(smem + h_late * A_SLOTS, smem + h_early * A_SLOTS, kk, buf);
        else
            read_frags(smem + h_early * A_SLOTS, smem + h_late * A_SLOTS, kk, buf);
    };
    auto ring_loop_rows = [&](auto shift_tag) {
        constexpr int SH = decltype(shift_tag)::value;
        static_assert(SH + NWIN <= KSTEPS && KSTEPS >= 3, "k step 2 carries the rows");
        constexpr int NVALU_T = B_BLOCKS * 16;  // dword selects of the transposes
        load_brow(0);
#pragma unroll
        for (int q = 0; q < JE; ++q) dma_e(q, 0, smem);
#pragma unroll
        for (int q = 0; q < JE; ++q) dma_e(q, min(1, nslabs - 1) * BK, smem + 2 * A_SLOTS);
        wait_vmcnt<2 * JE>();  // rows of slab 0
        write_brow(smem + A_SLOTS);
        load_brow(1);
        if (SH == 0) ring_window(0, 1, 3, 2, 4);  // DMA operand of slab 2
        wait_vmcnt<JE + NBL + (SH == 0 ? DMA_PER_WIN : 0)>();  // DMA operand of slab 0
        wait_lgkmcnt0();
        lds_barrier();
        frags_at(0, 1, 0, 0);
        int ha = 0;  // early half of slab s; its late half is ha + 1
        for (int s = 0; s < nslabs; ++s) {
            const int hb = wrap5(ha + 1), hna = wrap5(ha + 2), hnb = wrap5(ha + 3), hfa = wrap5(ha + 4);
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int cb = kk & 1;
                wait_lgkmcnt0();
                if (kk + 1 < KSTEPS) {
                    __builtin_amdgcn_sched_barrier(0);
                    frags_at(ha, hb, kk + 1, cb ^ 1);
                    const int win = kk + 1 - SH;
                    const bool has = win >= 0 && win < NWIN;
                    if (has) ring_window(win, s + 1, hnb, s + 2, hfa);
                    const int dmas = has ? dmas_in(win) : 0;
                    if (kk == 2) {
                        // one register buffer: slab s+1's rows go to LDS before the same
                        // registers take slab s+2's
                        wait_vmcnt<JE>();  // rows of slab s+1 (only the DMA of slab s+2 after them)
                        write_brow(smem + hnb * A_SLOTS);
                        load_brow(s + 2);
                        mfma_spread(cb, NREAD, dmas + NBL, NVALU_T, B_BLOCKS * 4);
                    } else {
                        mfma_woven(cb, NREAD, dmas);
                    }
                } else {
                    lds_barrier();  // slab s+1 published (its rows were written and waited for)
                    frags_at(hna, hnb, 0, cb ^ 1);
                    if (SH == 0) ring_window(0, s + 2, ha, s + 3, hb);
                    mfma_woven(cb, NREAD, SH == 0 ? dmas_in(0) : 0);
                }
            }
            ha = wrap5(ha + 2);
        }
    };
    if constexpr (RING == 5 && ANY_ROW) {
        if (STAGGER && wave >= NWAVES / 2)
            ring_loop_rows(std::integral_constant<int, STAGGER ? 1 : 0>{});
        else
            ring_loop_rows(std::integral_constant<int, 0>{});
    } else if constexpr (RING == 5) {
        if (STAGGER && wave >= NWAVES / 2)
            ring_loop(std::integral_constant<int, STAGGER ? 1 : 0>{});
        else
            ring_loop(std::integral_constant<int, 0>{});
    } else {
        if (STAGGER && wave >= NWAVES / 2)
            main_loop(std::integral_constant<int, STAGGER ? 1 : 0>{});
        else
            main_loop(std::integral_constant<int, 0>{});
    }
    wait_vmcnt<0>();  // no LDS DMA may still be in flight when the workgroup retires

    // Epilogue: accumulator v of a fragment lands at (row_lane + row_acc(v), lane % MF) of
    // its MF x MF block. Stores go through a buffer descriptor over the tile's BM rows of C:
    // one per-lane byte offset for the whole epilogue, the (i, j, v) part wave-uniform (the
    // launch checks that BM rows of C span less than 2^31 bytes). beta == 0 never reads C.
    // (past M, the descriptor drops the stores of the rows beyond; past N, lanes whose column
    // is beyond N get an offset past the descriptor's end, 2^31 > BM rows of C, so the
    // hardware drops those stores too)
    const rsrc_t c_rsrc = make_rsrc(C + (int64_t)m0 * ldc + n0, addr::desc_bytes(min(BM, M - m0), ldc, N - n0, 4));
    // (the lane index is recomputed from mbcnt so no thread-id register stays live across
    // the main loop)
    const int elane = __lane_id();
    const uint32_t lane_off = addr::c_lane_off<MF>(wm * WTM, wn * WTN, elane, ldc);
    uint32_t lane_off_j[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j)
        lane_off_j[j] = n0 + wn * WTN + j * MF + elane % MF < N ? lane_off : addr::kPastEnd;
    auto c_off = [&](int i, int j, int v) { return addr::c_acc_off<MF>(i, j, v, ldc); };
    if (beta != 0.0f) {
        // One row of fragments at a time: all of its C loads, then all of its stores. (Element
        // by element, each load waited for the stores before it, which may alias it: one memory
        // round trip per element. 8192x4096x8192 with beta = -0.5 took 609 us against 390 with
        // beta = 0; loaded a row of fragments at a time it takes 420.)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            float c[NI][F::NACC];
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v) c[j][v] = load_f32_buf(c_rsrc, lane_off_j[j], c_off(i, j, v));
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v)
                    store_f32_buf(c_rsrc, lane_off_j[j], c_off(i, j, v), fmaf(alpha, acc[i][j][v], beta * c[j][v]));
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v)
                    store_f32_buf(c_rsrc, lane_off_j[j], c_off(i, j, v), alpha * acc[i][j][v]);
    }
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int WINDOWS, int STAGGER, bool F16, int RING,
          int ROWS = 0, bool KTAIL = false, int MN = 0>
hipError_t launch_dma_cfg(const Problem &p, hipStream_t s) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    note_launch(reinterpret_cast<const void *>(
                    &bf16_mfma_dma_kernel<BM, BN, BK, WM, WN, MF, WINDOWS, STAGGER, F16, RING, ROWS, KTAIL, MN>),
                WM * WN * 64);
    hipLaunchKernelGGL((bf16_mfma_dma_kernel<BM, BN, BK, WM, WN, MF, WINDOWS, STAGGER, F16, RING, ROWS, KTAIL, MN>), dim3(tiles_m * tiles_n),
                       dim3(WM * WN * 64), 0, s, p.M, p.N, p.K, p.alpha, (const uint16_t *)p.A,
                       p.lda, (const uint16_t *)p.B, p.ldb, p.beta, p.C, p.ldc, tiles_m, tiles_n);
    return hipGetLastError();
}



#ifndef DMA_BM
#define DMA_BM 256
#define DMA_BN 256
#define DMA_BK 64
#define DMA_WM 2
#define DMA_WN 2
#endif
// DMA windows per slab and stagger, per fragment shape (tuned at 8192^3: one window right
// after the barrier, the second half of the waves one k step later)
#ifndef DMA_WIN32
#define DMA_WIN32 1
#define DMA_STAG32 1
#define DMA_WIN16 1
#define DMA_STAG16 1
#endif
// LDS layout per fragment shape: a ring of five half-stages for both (32x32x16: +3.5% at
// 8192^3 against two stages; 16x16x32 with the stagger: 1234 against 1045 TFLOP/s at 8192^3
// and 1173 against 985 at 4096^3, same box, interleaved)
#ifndef DMA_SMALL_WIN
#define DMA_SMALL_WIN 2
#define DMA_SMALL_STAG 0
#endif
#ifndef DMA_RING32
#define DMA_RING32 5
#endif
#ifndef DMA_RING16
#define DMA_RING16 5
#endif

template <bool F16, bool KTAIL>
hipError_t launch_dma_shape(const Problem &p, hipStream_t s, int shape, bool small) {
    // small: 128x128 tiles (64x64 per wave, 80 KB of LDS, two workgroups per CU), two DMA
    // windows per slab and no stagger (best of the four window / stagger settings that fit,
    // two or three windows with or without the stagger, measured at 2048x2048x8192,
    // 2048x1024x8192, 1536x1536x8192, 3000x2000x2000 and 2048x4096x4096: the others lost up
    // to 19%; one window needs more DMA issue slots per k step than the 4 MFMAs give)
    if (small) return launch_dma_cfg<128, 128, DMA_BK, 2, 2, 32, DMA_SMALL_WIN, DMA_SMALL_STAG, F16, 5, 0, KTAIL>(p, s);
    if (shape == 16)
        return launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_WM, DMA_WN, 16, DMA_WIN16, DMA_STAG16, F16, DMA_RING16, 0, KTAIL>(p, s);
    return launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_WM, DMA_WN, 32, DMA_WIN32, DMA_STAG32, F16, DMA_RING32, 0, KTAIL>(p, s);
}

}  // namespace

// Takes (and launches, status in *err) every problem whose operands are K-contiguous with
// K a multiple of 8 and 16-byte aligned rows (addr::kc_dma_takes); returns false, launching
// nothing, for any other. M and N may end inside a tile (the tile's descriptors stop at the
// last real row and column) and K inside the last slab (its chunks past K load as zeros). Up
// to 128 tiles of 256x256 (half a tile per CU) run on 128x128 tiles, which measured 24-76%
// faster there (2048x4096x4096: 986 against 769-799 TFLOP/s) and 5-10% slower from 144 tiles
// on (3072^3: 796 against 840), always with 32x32x16 fragments.
bool launch_bf16_mfma_dma(const Problem &p, hipStream_t s, const char **name, int shape, bool f16,
                          hipError_t *err) {
    const bool small = addr::dma_tile(p.M, p.N) == 128;
    if (!(addr::kc_dma_takes(p.M, p.N, p.K, p.lda, p.ldb, p.ldc) && aligned16(p.A) && aligned16(p.B) &&
          (shape == 32 || shape == 16)))
        return false;
    const bool ktail = p.K % DMA_BK != 0;
    const int kind = small ? 2 : shape == 16;  // 0: 256x256 32x32x16, 1: 256x256 16x16x32, 2: 128x128
#define REGTILE_DMA_NAME(elt, mf, bm, bn)                                                          \
    elt "_mfma" mf "_dma_" bm "x" bn "x" REGTILE_STR(DMA_BK) "_w" REGTILE_STR(DMA_WM) "x" REGTILE_STR(DMA_WN)
#define REGTILE_DMA_NAMES(elt)                                                                     \
    {{REGTILE_DMA_NAME(elt, "32x32x16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)),                 \
      REGTILE_DMA_NAME(elt, "32x32x16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)) "_ktail"},       \
     {REGTILE_DMA_NAME(elt, "16x16x32", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)),                 \
      REGTILE_DMA_NAME(elt, "16x16x32", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)) "_ktail"},       \
     {REGTILE_DMA_NAME(elt, "32x32x16", "128", "128"), REGTILE_DMA_NAME(elt, "32x32x16", "128", "128") "_ktail"}}
    static const char *const names[2][3][2] = {REGTILE_DMA_NAMES("bf16"), REGTILE_DMA_NAMES("f16")};
#undef REGTILE_DMA_NAMES
#undef REGTILE_DMA_NAME
    *name = names[f16][kind][ktail];
    if (f16)
        *err = ktail ? launch_dma_shape<true, true>(p, s, shape, small) : launch_dma_shape<true, false>(p, s, shape, small);
    else
        *err = ktail ? launch_dma_shape<false, true>(p, s, shape, small) : launch_dma_shape<false, false>(p, s, shape, small);
    return true;
}

// "t n": A stored K x M and B stored K x N, both M/N-contiguous. Both reach LDS by DMA in their
// own storage and feed the MFMAs through transposing LDS reads (the kernel template takes
// either operand that way; for "n n" and "t t" the register-row kernel measured level or
// faster, so only "t n" launches it). Up to 128 tiles of 256x256 run on 128x128 tiles.
// Takes (and launches, status in *err) a problem only when both operands' leading dimensions
// and column counts are multiples of 8 (so no 16-byte chunk straddles a descriptor that ends
// at the operand's last element), their rows are 16-byte aligned, and the offsets over all of
// K fit in 32 bits (addr::mn_dma_takes); returns false, launching nothing, otherwise. K and
// the tile grid may end anywhere.
bool launch_bf16_mfma_dma_mn(const Problem &p, hipStream_t s, const char **name, bool f16, hipError_t *err) {
    const bool small = addr::dma_tile(p.M, p.N) == 128;  // 128x128 tiles
    if (!(p.ta && !p.tb && DMA_RING32 == 5 && addr::mn_dma_takes(p.M, p.N, p.K, p.lda, p.ldb, p.ldc) &&
          aligned16(p.A) && aligned16(p.B)))
        return false;
    const bool ktail = p.K % DMA_BK != 0;
#define REGTILE_DMA_MN_NAME(elt, bm, bn)                                                           \
    elt "_mfma32x32x16_dma_tr_" bm "x" bn "x" REGTILE_STR(DMA_BK) "_w" REGTILE_STR(DMA_WM) "x"       \
        REGTILE_STR(DMA_WN) "_tn"
#define REGTILE_DMA_MN_PAIR(elt, bm, bn) {REGTILE_DMA_MN_NAME(elt, bm, bn), REGTILE_DMA_MN_NAME(elt, bm, bn) "_ktail"}
    static const char *const names[2][2][2] = {
        {REGTILE_DMA_MN_PAIR("bf16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)), REGTILE_DMA_MN_PAIR("bf16", "128", "128")},
        {REGTILE_DMA_MN_PAIR("f16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)), REGTILE_DMA_MN_PAIR("f16", "128", "128")}};
#undef REGTILE_DMA_MN_PAIR
#undef REGTILE_DMA_MN_NAME
    *name = names[f16][small][ktail];
    // small: the K-contiguous kernel's 128x128 set-up (two DMA windows per slab, no stagger)
#define REGTILE_MN_LAUNCH(F16_, KT_)                                                               \
    (small ? launch_dma_cfg<128, 128, DMA_BK, 2, 2, 32, 2, 0, F16_, 5, 0, KT_, 3>(p, s)             \
           : launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_WM, DMA_WN, 32, DMA_WIN32, DMA_STAG32, F16_, 5, 0, KT_, 3>(p, s))
    if (f16)
        *err = ktail ? REGTILE_MN_LAUNCH(true, true) : REGTILE_MN_LAUNCH(true, false);
    else
        *err = ktail ? REGTILE_MN_LAUNCH(false, true) : REGTILE_MN_LAUNCH(false, false);
    return true;
#undef REGTILE_MN_LAUNCH
}

// One operand M- or N-contiguous, the other K-contiguous: "n n" (A row-major, B stored K x N)
// or "t t" (A stored K x M, B stored N x K). The K-contiguous operand goes over LDS DMA, the
// other as 8-byte row runs through registers, transposed into the slab. Up to 128 tiles
// of 256x256 run on 128x128 tiles. Takes (and launches, status in *err) a problem only when
// K is a multiple of 8, the DMA operand's rows are 16-byte aligned within 32-bit tile offsets,
// and the row operand's leading dimension and column count are multiples of 4 with 8-byte
// aligned rows within 32-bit offsets over all of K (addr::rows_dma_takes); returns false,
// launching nothing, otherwise. M, N and K may end inside a tile.
bool launch_bf16_mfma_dma_rows(const Problem &p, hipStream_t s, const char **name, bool f16, hipError_t *err) {
    const bool nn = !p.ta && !p.tb, tt = p.ta && p.tb;
    const bool small = addr::dma_tile(p.M, p.N) == 128;  // 128x128 tiles, as in the K-contiguous kernel
    if (!((nn || tt) && DMA_RING32 == 5 && addr::rows_dma_takes(nn, p.M, p.N, p.K, p.lda, p.ldb, p.ldc) &&
          aligned16(nn ? p.A : p.B) && aligned8(nn ? p.B : p.A)))
        return false;
    const bool ktail = p.K % DMA_BK != 0;
#define REGTILE_DMA_ROWS_NAME(elt, bm, bn, lay)                                                   \
    elt "_mfma32x32x16_dma_" bm "x" bn "x" REGTILE_STR(DMA_BK) "_w" REGTILE_STR(DMA_WM) "x"        \
        REGTILE_STR(DMA_WN) "_" lay
#define REGTILE_DMA_ROWS_PAIR(elt, bm, bn, lay)                                                   \
    {REGTILE_DMA_ROWS_NAME(elt, bm, bn, lay), REGTILE_DMA_ROWS_NAME(elt, bm, bn, lay) "_ktail"}
#define REGTILE_DMA_ROWS_SIZE(elt, bm, bn)                                                        \
    {REGTILE_DMA_ROWS_PAIR(elt, bm, bn, "tt"), REGTILE_DMA_ROWS_PAIR(elt, bm, bn, "nn")}
    static const char *const names[2][2][2][2] = {
        {REGTILE_DMA_ROWS_SIZE("bf16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)),
         REGTILE_DMA_ROWS_SIZE("bf16", "128", "128")},
        {REGTILE_DMA_ROWS_SIZE("f16", REGTILE_STR(DMA_BM), REGTILE_STR(DMA_BN)),
         REGTILE_DMA_ROWS_SIZE("f16", "128", "128")}};
#undef REGTILE_DMA_ROWS_SIZE
#undef REGTILE_DMA_ROWS_PAIR
#undef REGTILE_DMA_ROWS_NAME
    *name = names[f16][small][nn][ktail];
    // small: the K-contiguous kernel's 128x128 set-up (two DMA windows per slab, no stagger)
#define REGTILE_ROWS_LAUNCH(F16_, ROWS_, KT_)                                                      \
    (small ? launch_dma_cfg<128, 128, DMA_BK, 2, 2, 32, 2, 0, F16_, 5, ROWS_, KT_>(p, s)            \
           : launch_dma_cfg<DMA_BM, DMA_BN, DMA_BK, DMA_WM, DMA_WN, 32, DMA_WIN32, DMA_STAG32, F16_, 5, ROWS_, KT_>(p, s))
    if (f16) {
        if (nn) *err = ktail ? REGTILE_ROWS_LAUNCH(true, 1, true) : REGTILE_ROWS_LAUNCH(true, 1, false);
        else *err = ktail ? REGTILE_ROWS_LAUNCH(true, 2, true) : REGTILE_ROWS_LAUNCH(true, 2, false);
    } else {
        if (nn) *err = ktail ? REGTILE_ROWS_LAUNCH(false, 1, true) : REGTILE_ROWS_LAUNCH(false, 1, false);
        else *err = ktail ? REGTILE_ROWS_LAUNCH(false, 2, true) : REGTILE_ROWS_LAUNCH(false, 2, false);
    }
    return true;
#undef REGTILE_ROWS_LAUNCH
}

}  // namespace regtile
