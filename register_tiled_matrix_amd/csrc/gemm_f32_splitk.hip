// gemm_f32_splitk.hip -- the fp32 register-tiled kernels for problems with few output tiles
// (tall-skinny or small M, N): split-K inside the workgroup.
//
// With 128x128 tiles a 16384 x 128 output is only 128 workgroups for 256 CUs, half a wave per
// SIMD. Here a workgroup owns a smaller tile and each of its NW waves accumulates that whole
// tile over its own share of K, with the register micro-tile of the square kernel
// ("Understanding Register Tiling" (blog.csdn.net/sweet_ran), the key loop: regA / regB per
// k, TM x TN FMAs per k held in registers; "寄存器Tiling跨架构解析" section 2.4 / 7.2: trade
// tile size against the number of resident waves). Five shapes:
//   * 32x32 tile, 8 waves, 4x4 micro-tiles, BK 16 (splitk8, problems of fewer than 64 tiles
//     of 64x64; the first 256 threads run the epilogue);
//   * 64x64 tile, 8 waves, 8x8 micro-tiles, BK 16 (splitk8, below 448 such tiles: two waves
//     per SIMD where the 4-wave form would leave one);
//   * 64x64 tile, 4 waves, 8x8 micro-tiles, BK 16 (splitk4);
//   * 64x128 tile, 8 waves, 8x16 micro-tiles (the square kernel's), BK 8 (splitk8): one
//     workgroup of two waves per SIMD per CU, and three quarters of the LDS reads per FMA of
//     8x8;
//   * 64x96 tile, 8 waves, 8x12 micro-tiles, BK 8: the same with three column groups, for
//     shapes whose 64x128 tiles fill only part of a round of 256 workgroups.
// The partial tiles are summed through LDS in a fixed order, so results are deterministic;
// the summation order differs from the square kernel's single k sweep.
//
// Per wave: 64 lanes as an 8x8 grid, lane micro-tile rows r0 + 32 g + {0..3} for g < TM/4 and
// columns c0 + 32 g + {0..3} for g < TN/4 (every wave-wide 16-byte fragment read is one
// contiguous 128-byte run). Each wave stages its own A slab (k-major, padded) and B slab in
// its own two LDS buffers. No wave reads another wave's buffers, so the main loop needs no
// workgroup barrier: a wave writes buffer (s+1) & 1 only after the fragments it read from that
// buffer one slab earlier have been consumed by its own FMAs.
#include "regtile_internal.h"

namespace regtile {

namespace {

constexpr int APAD = 4;
// 1: one LDS wait per k step in the split-K loop (the compiler otherwise waits fragment by
// fragment); 0: the compiler's waits
#ifndef SPLIT_ONE_WAIT
#define SPLIT_ONE_WAIT 1
#endif
#ifndef SPLIT_PAIR_SWAP
#define SPLIT_PAIR_SWAP 1
#endif
#ifndef SPLIT96_BK
#define SPLIT96_BK 8
#endif
#ifndef SPLIT96_APAD
#define SPLIT96_APAD 4
#endif

#ifndef SPLIT96_DEPTH
#define SPLIT96_DEPTH 1
#endif
// 1: wave w runs slabs w, w + NW, w + 2 NW, ... of K (the waves of a workgroup sweep K side by
// side, so at any time they read neighbouring k of the same A rows and share its cache lines);
// 0: wave w runs one contiguous range of slabs
#ifndef SPLIT_INTERLEAVE
#define SPLIT_INTERLEAVE 1
#endif

template <int NW_, int TM_, int TN_, int BK_, int DEPTH_ = 1, int PAD_ = APAD>
struct SplitCfg {
    // DEPTH: slabs of global loads in flight ahead of the slab being computed (1 or 2; 2 holds
    // a second set of staging registers)
    static constexpr int NW = NW_, TM = TM_, TN = TN_, BK = BK_, DEPTH = DEPTH_;
    static_assert(DEPTH == 1 || DEPTH == 2, "one or two slabs of loads in flight");
    static constexpr int NT = NW * 64;
    static constexpr int TILE_M = 8 * TM, TILE_N = 8 * TN;  // 8 x 8 lanes per wave
    static constexpr int AS = TILE_M + PAD_;                // A slab row stride (floats), k-major
    static constexpr int NA4 = TILE_M * BK / 256;           // A float4 per lane per slab
    static constexpr int NB4 = BK * TILE_N / 256;           // B float4 per lane per slab
    static constexpr int NPART = NW < 4 ? NW : 4;           // partial tiles held in LDS at once
    // epilogue columns per thread (at least one float4: with more threads than float4 of the
    // tile, only the first ET threads run the epilogue)
    static constexpr int SW = TILE_M * TILE_N / NT < 4 ? 4 : TILE_M * TILE_N / NT;
    static constexpr int ET = TILE_M * TILE_N / SW;         // threads that run the epilogue
    static_assert((TM == 4 || TM == 8) && (TN == 4 || TN == 8 || TN == 12 || TN == 16),
                  "micro-tile rows in one or two groups of 4");
    static_assert(SW % 4 == 0 && TILE_N % SW == 0, "whole float4 strips in the epilogue");
    static_assert(NW == 4 || NW == 8, "four waves, or eight summed pairwise first");
    static_assert(NA4 >= 1 && NB4 >= 1 && TILE_M * BK % 256 == 0 && BK * TILE_N % 256 == 0,
                  "whole float4 per lane");
    struct alignas(16) WaveStage {
        float a[BK][AS];
        float b[BK][TILE_N];
    };
    struct alignas(16) Smem {
        union {
            WaveStage st[NW][2];
            float part[NPART][TILE_M][TILE_N + 4];  // partial tiles after the main loop (padded)
        };
    };
};
using Split4 = SplitCfg<4, 8, 8, 16>;
using Split8t = SplitCfg<8, 4, 4, 16>;  // 32x32 tiles for problems of a few 64x64 tiles
using Split8s = SplitCfg<8, 8, 8, 16>;  // 64x64 tiles, 8 waves: two waves per SIMD on one tile per CU
using Split8 = SplitCfg<8, 8, 16, 8>;
using Split8n96 = SplitCfg<8, 8, 12, SPLIT96_BK, SPLIT96_DEPTH, SPLIT96_APAD>;  // 64x96 tiles: 1000 x 1500 is 256 of them

template <bool GUARD, bool VEC>
__device__ __forceinline__ float4 load4(const float *__restrict__ p, bool row_ok, int cols_left) {
    if (!GUARD) {
        if (VEC) return *reinterpret_cast<const float4 *>(p);
        return load_f4_any(p);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok) {
        if (cols_left >= 4) {
            v = VEC ? *reinterpret_cast<const float4 *>(p) : load_f4_any(p);
        } else {
            if (cols_left > 0) v.x = p[0];
            if (cols_left > 1) v.y = p[1];
            if (cols_left > 2) v.z = p[2];
            if (cols_left > 3) v.w = p[3];
        }
    }
    return v;
}

// GUARD: bounds checks on every load (ragged M/N, or K not a multiple of NW*BK).
template <class CFG, bool GUARD, bool VEC_A, bool VEC_B, bool VEC_C>
__global__ __launch_bounds__(CFG::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void f32_splitk_kernel(
    int M, int N, int K, float alpha, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int slabs_per_wave) {
    constexpr int NW = CFG::NW, TM = CFG::TM, TN = CFG::TN, BK = CFG::BK, NT = CFG::NT;
    constexpr int TILE_M = CFG::TILE_M, TILE_N = CFG::TILE_N, AS = CFG::AS;
    constexpr int NA4 = CFG::NA4, NB4 = CFG::NB4, NPART = CFG::NPART;
    constexpr int AQ = BK / 4, BQ = TILE_N / 4;  // float4 per A row / per B row of a slab
    __shared__ typename CFG::Smem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r0 = (lane >> 3) * 4, c0 = (lane & 7) * 4;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * TILE_M, n0 = tn * TILE_N;
    // This wave's slabs: slab t of the wave starts at k = kslab(t). Interleaved, wave w runs
    // slabs w, w + NW, ... of the K sweep and every load stops at K; in ranges, it runs a
    // contiguous range [kb, ke). Waves may run different slab counts: the main loop has no
    // workgroup barrier.
    const int nslabs = (K + BK - 1) / BK;
    const int kb = SPLIT_INTERLEAVE ? 0 : wave * slabs_per_wave * BK;
    const int ke = SPLIT_INTERLEAVE ? K : min(K, kb + slabs_per_wave * BK);
    const int spw_w = SPLIT_INTERLEAVE ? (nslabs > wave ? (nslabs - wave + NW - 1) / NW : 0)
                                       : (ke > kb ? (ke - kb + BK - 1) / BK : 0);
    auto kslab = [&](int t) { return SPLIT_INTERLEAVE ? (t * NW + wave) * BK : kb + t * BK; };

    // Staging: float4 q of the A slab (TILE_M rows x BK k) is row q / AQ, k (q % AQ) * 4;
    // float4 q of the B slab (BK k x TILE_N columns) is k q / BQ, column (q % BQ) * 4. With
    // DEPTH 2 a second register set (ra2, rb2) holds the slab after next.
    //
    // Edges: an A row past M reads row M - 1 instead, and a B column chunk wholly past N reads
    // the tile's first chunk instead; both only feed outputs that are never stored, so they
    // need no zeros. What must be zero is every k at or past ke (other waves' k, or past K),
    // and the columns past N of a chunk that straddles N (its real columns are kept). A slab
    // wholly inside [kb, ke) with no straddling chunk in the wave therefore takes plain vector
    // loads; only the others take the element-checked loads.
    const float *a_src[NA4];
    const float *b_src[NB4];
    int b_cols_left[NB4];
    bool straddle = false;
#pragma unroll
    for (int i = 0; i < NA4; ++i) {
        const int q = lane + 64 * i;
        const int ar = q / AQ, ak = (q % AQ) * 4;
        const int row = GUARD ? min(m0 + ar, M - 1) : m0 + ar;
        a_src[i] = A + (int64_t)row * lda + ak;
    }
#pragma unroll
    for (int i = 0; i < NB4; ++i) {
        const int q = lane + 64 * i;
        const int bk = q / BQ, bc = (q % BQ) * 4;
        const int col = GUARD && n0 + bc >= N ? n0 : n0 + bc;
        b_src[i] = B + (int64_t)bk * ldb + col;
        b_cols_left[i] = N - col;
        straddle |= GUARD && N - col < 4;
    }
    // (wave-uniform: one vote for the whole kernel)
    const bool any_straddle = GUARD && __any(straddle);
    float4 ra[NA4], rb[NB4], ra2[NA4], rb2[NB4];
    auto load_into = [&](int k0, float4 (&xa)[NA4], float4 (&xb)[NB4]) {
        if (!GUARD || (!any_straddle && k0 + BK <= ke)) {
#pragma unroll
            for (int i = 0; i < NA4; ++i) xa[i] = load4<false, VEC_A>(a_src[i] + k0, true, 4);
#pragma unroll
            for (int i = 0; i < NB4; ++i) xb[i] = load4<false, VEC_B>(b_src[i] + (int64_t)k0 * ldb, true, 4);
        } else {
#pragma unroll
            for (int i = 0; i < NA4; ++i) {
                const int ak = ((lane + 64 * i) % AQ) * 4;
                xa[i] = load4<true, VEC_A>(a_src[i] + k0, true, ke - (k0 + ak));
            }
#pragma unroll
            for (int i = 0; i < NB4; ++i) {
                const int bk = (lane + 64 * i) / BQ;
                xb[i] = load4<true, VEC_B>(b_src[i] + (int64_t)k0 * ldb, k0 + bk < ke, b_cols_left[i]);
            }
        }
    };
    auto load_slab = [&](int k0) { load_into(k0, ra, rb); };
    auto store_from = [&](int buf, const float4 (&xa)[NA4], const float4 (&xb)[NB4]) {
        auto &w = sm.st[wave][buf];
#pragma unroll
        for (int i = 0; i < NA4; ++i) {
            const int q = lane + 64 * i;
            const int ar = q / AQ, ak = (q % AQ) * 4;
            w.a[ak + 0][ar] = xa[i].x;
            w.a[ak + 1][ar] = xa[i].y;
            w.a[ak + 2][ar] = xa[i].z;
            w.a[ak + 3][ar] = xa[i].w;
        }
#pragma unroll
        for (int i = 0; i < NB4; ++i) {
            const int q = lane + 64 * i;
            const int bk = q / BQ, bc = (q % BQ) * 4;
            *reinterpret_cast<float4 *>(&w.b[bk][bc]) = xb[i];
        }
    };
    auto store_slab = [&](int buf) { store_from(buf, ra, rb); };

    float acc[TM][TN];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[m][n] = 0.0f;

    constexpr int MG = TM / 4, NG = TN / 4;  // row and column groups of 4, 32 apart
    auto compute_slab = [&](int buf) {
        const float *sa = &sm.st[wave][buf].a[0][0] + r0;
        const float *sb = &sm.st[wave][buf].b[0][0] + c0;
        float4 fa[2][MG], fb[2][NG];
#pragma unroll
        for (int g = 0; g < MG; ++g) fa[0][g] = *reinterpret_cast<const float4 *>(sa + 32 * g);
#pragma unroll
        for (int g = 0; g < NG; ++g) fb[0][g] = *reinterpret_cast<const float4 *>(sb + 32 * g);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const int cb = k & 1, nb = cb ^ 1;
            if (k + 1 < BK) {
#pragma unroll
                for (int g = 0; g < MG; ++g)
                    fa[nb][g] = *reinterpret_cast<const float4 *>(sa + (k + 1) * AS + 32 * g);
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    fb[nb][g] = *reinterpret_cast<const float4 *>(sb + (k + 1) * TILE_N + 32 * g);
                // one wait for all of step k's fragments: only step k+1's reads may still be in
                // flight (LDS operations of a wave complete in order, the slab's stores included)
                if constexpr (SPLIT_ONE_WAIT) wait_lgkmcnt<MG + NG>();
            } else if constexpr (SPLIT_ONE_WAIT) {
                wait_lgkmcnt<0>();
            }
            if constexpr (SPLIT_ONE_WAIT) __builtin_amdgcn_sched_barrier(0);  // no FMA above the wait
            float a_[TM];
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                a_[4 * g + 0] = fa[cb][g].x;
                a_[4 * g + 1] = fa[cb][g].y;
                a_[4 * g + 2] = fa[cb][g].z;
                a_[4 * g + 3] = fa[cb][g].w;
            }
            float b_[TN];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                b_[4 * g + 0] = fb[cb][g].x;
                b_[4 * g + 1] = fb[cb][g].y;
                b_[4 * g + 2] = fb[cb][g].z;
                b_[4 * g + 3] = fb[cb][g].w;
            }
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n) acc[m][n] = fmaf(a_[m], b_[n], acc[m][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Each wave runs its own slabs; the last slab of the sweep may reach past ke = K (loads
    // past ke are zeros).
    const int spw = spw_w;
    if constexpr (CFG::DEPTH == 1) {
        if (spw > 0) {
            load_slab(kslab(0));
            store_slab(0);
            for (int s = 0; s + 1 < spw; ++s) {
                load_slab(kslab(s + 1));
                compute_slab(s & 1);
                store_slab((s + 1) & 1);
            }
            compute_slab((spw - 1) & 1);
        }
    } else {
        // Two register sets, two LDS buffers. Slab t's loads go out while slab t - 2 is
        // computed and reach LDS after slab t - 1 has been: two slabs of latency covered.
        // Set (ra, rb) carries the even slabs and buffer 0, set (ra2, rb2) the odd slabs and
        // buffer 1; the loop body is one pair of slabs so both sets stay in fixed registers.
        if (spw > 0) {
            load_into(kslab(0), ra, rb);
            if (spw > 1) load_into(kslab(1), ra2, rb2);
            store_from(0, ra, rb);
            int s = 0;
            for (; s + 2 < spw; s += 2) {
                // slab s (even): buffer 0; slab s + 1 waits in (ra2, rb2)
                load_into(kslab(s + 2), ra, rb);
                compute_slab(0);
                store_from(1, ra2, rb2);
                // slab s + 1 (odd): buffer 1; slab s + 2 waits in (ra, rb)
                if (s + 3 < spw) load_into(kslab(s + 3), ra2, rb2);
                compute_slab(1);
                store_from(0, ra, rb);
            }
            // the last one or two slabs: s even, s + 1 < spw iff a slab waits in (ra2, rb2)
            compute_slab(0);
            if (s + 1 < spw) {
                store_from(1, ra2, rb2);
                compute_slab(1);
            }
        }
    }
    // The epilogue's strip of C (beta != 0) is read now, so its latency overlaps the reduction
    // below rather than following it: thread t owns row t / (TILE_N / SW), columns
    // (t % (TILE_N / SW)) * SW .. +SW-1 (SW = 16, or 12 for 96-column tiles).
    constexpr int SW = CFG::SW, TPR = TILE_N / SW, ET = CFG::ET;  // strip width, threads per row
    static_assert(ET == TILE_M * TPR && ET <= NT, "one strip per epilogue thread");
    const bool epi = ET == NT || tid < ET;
    const int row = (epi ? tid : 0) / TPR, col0 = (tid % TPR) * SW;
    const int grow = m0 + row;
    float4 cold[SW / 4];
    if (epi && beta != 0.0f && (!GUARD || grow < M)) {
        const float *crow_in = C + (int64_t)grow * ldc + n0 + col0;
#pragma unroll
        for (int c4 = 0; c4 < SW / 4; ++c4) {
            const int gcol = n0 + col0 + c4 * 4;
            if (VEC_C && (!GUARD || gcol + 3 < N)) {
                cold[c4] = *reinterpret_cast<const float4 *>(crow_in + c4 * 4);
            } else {
                float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (!GUARD || gcol + u < N) e[u] = crow_in[c4 * 4 + u];
                cold[c4] = make_float4(e[0], e[1], e[2], e[3]);
            }
        }
    }
    __syncthreads();  // all waves are done with their stages: the union turns into partials

    // Partial tiles sit in LDS with the columns of each pair swapped (SWAP). The float4 that
    // writes acc[m][4g..4g+3] makes the compiler give those four accumulators one aligned
    // register quad; in this order acc[m][n] lands in an odd register for even n. The
    // fragments' quads put a[m] and b[n] in even registers for even m and n, so no FMA then
    // reads three even registers, a form that issues at two thirds of the FMA rate.
    constexpr bool SWAP = SPLIT_PAIR_SWAP;
    auto write_part = [&](int slot) {
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const int row = r0 + (m / 4) * 32 + m % 4;
#pragma unroll
            for (int g = 0; g < NG; ++g)
                *reinterpret_cast<float4 *>(&sm.part[slot][row][c0 + 32 * g]) =
                    SWAP ? make_float4(acc[m][4 * g + 1], acc[m][4 * g], acc[m][4 * g + 3], acc[m][4 * g + 2])
                         : make_float4(acc[m][4 * g], acc[m][4 * g + 1], acc[m][4 * g + 2], acc[m][4 * g + 3]);
        }
    };
    if constexpr (NW == 8) {
        // waves 4..7 hand their partials to waves 0..3, which add them (acc_w + acc_{w+4}) and
        // write the sum back into the same slot: slot w is touched only by waves w + 4 (before
        // the barrier) and w (after it), so no second barrier is needed before that write
        if (wave >= 4) write_part(wave - 4);
        __syncthreads();
        if (wave < 4) {
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                const int row = r0 + (m / 4) * 32 + m % 4;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const float4 p = *reinterpret_cast<const float4 *>(&sm.part[wave][row][c0 + 32 * g]);
                    acc[m][4 * g + (SWAP ? 1 : 0)] += p.x;
                    acc[m][4 * g + (SWAP ? 0 : 1)] += p.y;
                    acc[m][4 * g + (SWAP ? 3 : 2)] += p.z;
                    acc[m][4 * g + (SWAP ? 2 : 3)] += p.w;
                }
            }
            write_part(wave);
        }
    } else {
        write_part(wave);
    }
    __syncthreads();

    // Fixed-order sum of the NPART partials and epilogue on the strip read above.
    if (!epi || (GUARD && grow >= M)) return;
    float *crow = C + (int64_t)grow * ldc;
#pragma unroll
    for (int c4 = 0; c4 < SW / 4; ++c4) {
        const int col = col0 + c4 * 4;
        float4 s = *reinterpret_cast<const float4 *>(&sm.part[0][row][col]);
#pragma unroll
        for (int w = 1; w < NPART; ++w) {
            const float4 p = *reinterpret_cast<const float4 *>(&sm.part[w][row][col]);
            s.x += p.x;
            s.y += p.y;
            s.z += p.z;
            s.w += p.w;
        }
        if (SWAP) s = make_float4(s.y, s.x, s.w, s.z);
        const int gcol = n0 + col;
        float *c = crow + gcol;
        float4 v;
        if (beta == 0.0f) {  // C is never read
            v = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
        } else {
            const float4 old = cold[c4];
            v = make_float4(fmaf(alpha, s.x, beta * old.x), fmaf(alpha, s.y, beta * old.y),
                            fmaf(alpha, s.z, beta * old.z), fmaf(alpha, s.w, beta * old.w));
        }
        if (VEC_C && (!GUARD || gcol + 3 < N)) {
            *reinterpret_cast<float4 *>(c) = v;
        } else {
            const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!GUARD || gcol + e < N) c[e] = sv[e];
        }
    }
}

template <class CFG, bool G, bool VA, bool VB, bool VC>
hipError_t launch_variant(const Problem &p, hipStream_t s, int tm, int tn, int spw) {
    note_launch(reinterpret_cast<const void *>(&f32_splitk_kernel<CFG, G, VA, VB, VC>), CFG::NT);
    hipLaunchKernelGGL((f32_splitk_kernel<CFG, G, VA, VB, VC>), dim3(tm * tn), dim3(CFG::NT), 0, s,
                       p.M, p.N, p.K, p.alpha, (const float *)p.A, p.lda, (const float *)p.B,
                       p.ldb, p.beta, p.C, p.ldc, tm, tn, spw);
    return hipGetLastError();
}
template <class CFG, bool G, bool VA, bool VB>
hipError_t pick_c(const Problem &p, hipStream_t s, int tm, int tn, int spw, bool vc) {
    return vc ? launch_variant<CFG, G, VA, VB, true>(p, s, tm, tn, spw)
              : launch_variant<CFG, G, VA, VB, false>(p, s, tm, tn, spw);
}
template <class CFG, bool G, bool VA>
hipError_t pick_b(const Problem &p, hipStream_t s, int tm, int tn, int spw, bool vb, bool vc) {
    return vb ? pick_c<CFG, G, VA, true>(p, s, tm, tn, spw, vc)
              : pick_c<CFG, G, VA, false>(p, s, tm, tn, spw, vc);
}
template <class CFG>
hipError_t launch_cfg(const Problem &p, hipStream_t s, const char **name, const char *base,
                      const char *guarded) {
    const int tiles_m = (p.M + CFG::TILE_M - 1) / CFG::TILE_M;
    const int tiles_n = (p.N + CFG::TILE_N - 1) / CFG::TILE_N;
    const int nslabs = (p.K + CFG::BK - 1) / CFG::BK;
    const int spw = (nslabs + CFG::NW - 1) / CFG::NW;  // slabs per wave
    // Interleaved slabs need the element checks only for a partial last slab; ranges also
    // for a K that does not fill NW equal ranges.
    const bool guard = (p.M % CFG::TILE_M) != 0 || (p.N % CFG::TILE_N) != 0 ||
                       (p.K % ((SPLIT_INTERLEAVE ? 1 : CFG::NW) * CFG::BK)) != 0;
    const bool va = (p.lda % 4) == 0 && aligned16(p.A);
    const bool vb = (p.ldb % 4) == 0 && aligned16(p.B);
    const bool vc = (p.ldc % 4) == 0 && aligned16(p.C);
    *name = guard ? guarded : base;
    if (guard)
        return va ? pick_b<CFG, true, true>(p, s, tiles_m, tiles_n, spw, vb, vc)
                  : pick_b<CFG, true, false>(p, s, tiles_m, tiles_n, spw, vb, vc);
    return va ? pick_b<CFG, false, true>(p, s, tiles_m, tiles_n, spw, vb, vc)
              : pick_b<CFG, false, false>(p, s, tiles_m, tiles_n, spw, vb, vc);
}

}  // namespace

// The 8-wave kernel runs one workgroup per CU, so the tile count in rounds of 256 workgroups
// times the tile's area estimates its time. 64x96 tiles (8x12 micro-tiles) win where they fill
// a round that 64x128 tiles leave partly idle (1000 x 1500: 256 tiles against 192).
static int64_t tiles_64(const Problem &p) { return (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64); }

static bool split8_prefers_96(int M, int N) {
    const int64_t tm64 = (M + 63) / 64;
    const int64_t t128 = tm64 * ((N + 127) / 128), t96 = tm64 * ((N + 95) / 96);
    return ((t96 + 255) / 256) * 96 < ((t128 + 255) / 256) * 128;
}

hipError_t launch_f32_splitk(const Problem &p, hipStream_t s, const char **name) {
    // Fewer than 64 tiles of 64x64 (a quarter of the CUs): 32x32 tiles of 4x4 micro-tiles, so
    // that four times as many workgroups share the work, each split over eight waves (256^3:
    // 64 workgroups, each wave 512 FMAs per lane against 4096 on a 64x64 tile; 6.8 us against
    // 7.7 with four waves per tile and 15.7 on 64x64 tiles).
    if (tiles_64(p) < 64)
        return launch_cfg<Split8t>(p, s, name, "f32_regtile_splitk8_32x32x16_4x4",
                                   "f32_regtile_splitk8_32x32x16_4x4_guard");
    // 8 waves x 8x16 once 64x128 tiles give most CUs a workgroup (two waves per SIMD), unless
    // the 4-wave kernel's 64x64 tiles already fill the chip and K is short enough that the
    // 8-wave kernel's longer reduction does not pay (measured on 13 row-major shapes with
    // 64 <= K <= 8192; the 8-wave kernel lost at 16384 x 128 x 1024 and won at x 4096).
    const int64_t tm64 = (p.M + 63) / 64;
    const int64_t t128 = tm64 * ((p.N + 127) / 128), t64 = tm64 * ((p.N + 63) / 64);
    if (t128 >= 192 && (p.K >= 1280 || t64 < 448)) {
        if (split8_prefers_96(p.M, p.N))
            return launch_cfg<Split8n96>(p, s, name, "f32_regtile_splitk8_64x96x8_8x12",
                                         "f32_regtile_splitk8_64x96x8_8x12_guard");
        return launch_cfg<Split8>(p, s, name, "f32_regtile_splitk8_64x128x8_8x16",
                                  "f32_regtile_splitk8_64x128x8_8x16_guard");
    }
    // Below 448 tiles of 64x64 the 4-wave kernel leaves most CUs with one workgroup, one wave
    // per SIMD; eight waves per 64x64 tile restore two (1024^3: 47.9 -> 68.9 TFLOP/s,
    // 1024x1024x8192: 59.6 -> 89.7, 768x768x4096: 33.3 -> 55.6 in same-box A/B runs).
    if (t64 < 448)
        return launch_cfg<Split8s>(p, s, name, "f32_regtile_splitk8_64x64x16_8x8",
                                   "f32_regtile_splitk8_64x64x16_8x8_guard");
    return launch_cfg<Split4>(p, s, name, "f32_regtile_splitk4_64x64x16_8x8",
                              "f32_regtile_splitk4_64x64x16_8x8_guard");
}

}  // namespace regtile
