// gemm_f32_regtile.hip -- rung 2 of the ladder: the fp32 register-tiled SIMT kernel.
//
// Three-level tiling ("寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507) section 1.1: a
// 128x128 block tile per workgroup of 256 threads, an 8x8 micro-tile per thread, 64 FMAs per
// k step held entirely in registers), here with a TM x TN micro-tile (default 8 x 16):
//   HBM -> LDS      a BM x BK slab of A (stored k-major, i.e. transposed) and a BK x BN slab
//                   of B per stage, two stages (the next slab's global loads are in flight
//                   while the current slab is consumed; section 6.3's prefetch, done here
//                   as double-buffered LDS plus register staging);
//   LDS -> VGPR     per k: regA[TM] (TM/4 16-byte reads of a column of the A slab) and
//                   regB[TN] (TN/4 16-byte reads of a row of the B slab) -- "Understanding
//                   Register Tiling" (blog.csdn.net/sweet_ran), the key loop;
//   VGPR FMA        acc[TM][TN] += regA[m] * regB[n]: TM*TN independent fp32 FMAs per k.
// LDS reads per FMA: (TM + TN) / (TM * TN) floats (0.19 for 8x16, 0.25 for 8x8), against 2
// for the one-output-per-thread kernel (the three-version comparison on the same page).
//
// Wave64 mapping. The 256 threads are 4 waves in a 2x2 grid; each wave's 64 lanes form an
// 8x8 grid, so the workgroup tile is BM = 16 TM by BN = 16 TN. A lane's rows are
// r0 + 32 g + {0..3} (g < TM/4) and its columns c0 + 32 h + {0..3} (h < TN/4): the groups of
// 4 make the 8 distinct 16-byte fragment addresses of one wave-wide read a single contiguous
// 128-byte run (all banks once, the rest broadcasts), so fragment reads are free of bank
// conflicts (section 1.2/7.3 of the same page: the register layout decides the LDS access
// pattern). TM, TN, BK and waves per SIMD are compile-time choices (F32_TM, F32_TN, F32_BK,
// F32_WAVES_PER_EU) so the micro-tile / occupancy trade of sections 2.4 and 7.2 can be swept.
//
// Every output accumulates fmaf over k in natural order, like rungs 0 and 1, so the three
// fp32 rungs agree bitwise.
#include "regtile_internal.h"

namespace regtile {

namespace {

// Kernel configurations (TM, TN, BK, waves per SIMD). The square one is the default
// register-tiled kernel; the small one (64x64 tiles) serves problems with few 128x256 tiles.
// The F32_* macros exist so other values can be built for the micro-tile sweep.
#ifndef F32_TN
#define F32_TN 16
#endif
#ifndef F32_TM
#define F32_TM 8
#endif
#ifndef F32_BK
#define F32_BK 16
#endif
#ifndef F32_EARLY_STORE
#define F32_EARLY_STORE 1
#endif
// 1: the FMAs of a k step walk the micro-tile row by row in alternating column order
// (consecutive FMAs always share a source register); 0: row by row, left to right
#ifndef F32_SNAKE
#define F32_SNAKE 0
#endif
#ifndef F32_WAVES_PER_EU
#define F32_WAVES_PER_EU 2
#endif
// LDS stages of A and B slabs: 2 (double buffering), 1 (one stage; the next slab waits in
// registers and is stored between two barriers) or 3 (a slab is stored two slabs before the one
// that last read its stage)
#ifndef F32_STAGES
#define F32_STAGES 2
#endif
struct SquareCfg {
    static constexpr int TM = F32_TM, TN = F32_TN, BK = F32_BK, WAVES = F32_WAVES_PER_EU,
                         STAGES = F32_STAGES;
};
struct SmallCfg {
    static constexpr int TM = 4, TN = 4, BK = 32, WAVES = 4, STAGES = 2;
};

constexpr int NT = 256;
typedef float quad_t __attribute__((__vector_size__(4 * sizeof(float))));  // one VGPR quad
constexpr int APAD = 4;  // A slab row stride BM + 4 floats: transposed stores hit 32 banks per half-wave

// TM x TN micro-tile per lane: TM rows in TM / 4 groups of 4 (32 rows apart), TN columns in
// TN / 4 groups of 4 (32 columns apart). A wave is an 8x8 grid of lanes, 4 waves in 2x2, so
// the workgroup tile is 16 TM x 16 TN.
template <int TM, int TN>
struct Shape {
    static_assert((TM == 4 || TM == 8 || TM == 16) && (TN == 4 || TN == 8 || TN == 16),
                  "micro-tiles of 4, 8 or 16 rows and columns");
    static constexpr int MG = TM / 4, NG = TN / 4, BM = 16 * TM, BN = 16 * TN;
};

// B rows get the same padding when B is staged by transposed stores (B stored N x K).
template <int BM, int BN, int BK, int BPAD, int ST>
struct alignas(16) Smem {
    float a[ST][BK][BM + APAD];
    float b[ST][BK][BN + BPAD];
};

// Global -> register staging of one slab. A: BM x BK as BK/4 float4 chunks per row;
// B: BK x BN as BN/4 float4 chunks per row. Each thread owns BK/8 chunks of each.
template <bool EDGE, bool VEC>
__device__ __forceinline__ float4 load4_rowwise(const float *__restrict__ p, int rows_left,
                                                int cols_left) {
    // p points at element (row, col) of a row-major matrix; rows_left = rows remaining from
    // this row (> 0 means in range), cols_left = columns remaining from col.
    if (!EDGE) {
        if (VEC) return *reinterpret_cast<const float4 *>(p);
        return load_f4_any(p);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rows_left > 0) {
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

// TA: A is stored K x M row-major (op(A) = A^T of the storage); TB: B is stored N x K.
template <class CFG, bool TA, bool TB, bool EDGE, bool VEC_A, bool VEC_B, bool VEC_C>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(CFG::WAVES, CFG::WAVES))) void f32_regtile_kernel(int M, int N, int K, float alpha,
                                                         const float *__restrict__ A, int64_t lda,
                                                         const float *__restrict__ B, int64_t ldb,
                                                         float beta, float *__restrict__ C,
                                                         int64_t ldc, int tiles_m, int tiles_n) {
    constexpr int TM = CFG::TM, TN = CFG::TN, BK = CFG::BK;
    typedef Shape<TM, TN> S;
    constexpr int MG = S::MG, NG = S::NG, BM = S::BM, BN = S::BN;
    static_assert(BK % 4 == 0 && (BM * BK) % (4 * NT) == 0 && (BN * BK) % (4 * NT) == 0,
                  "every thread stages whole float4 chunks");
    constexpr int CH = BM * BK / (4 * NT);   // A float4 chunks per thread per slab
    constexpr int CHB = BK * BN / (4 * NT);  // B float4 chunks per thread per slab
    constexpr int BPAD = TB ? APAD : 0;
    constexpr int BLD = BN + BPAD;           // LDS row stride of the B slab
    constexpr int ST = CFG::STAGES;
    static_assert(ST >= 1 && ST <= 3, "one to three LDS stages");
    __shared__ Smem<BM, BN, BK, BPAD, ST> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r0 = (wave >> 1) * (8 * TM) + (lane >> 3) * 4;
    const int c0 = (wave & 1) * (8 * TN) + (lane & 7) * 4;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Staging chunks: float4 chunk q = tid + NT*i of a slab, read along the operand's
    // contiguous dimension. A (BM x BK): stored M x K -> (m, k) = (q / (BK/4), 4 (q % (BK/4)));
    // stored K x M -> (k, m) = (q / (BM/4), 4 (q % (BM/4))). B (BK x BN): stored K x N ->
    // (k, n) = (q / (BN/4), 4 (q % (BN/4))); stored N x K -> (n, k) = (q / (BK/4), 4 (q % (BK/4))).
    // a_m/a_k (b_k/b_n) name the first element of the chunk in the tile.
    int a_m[CH], a_k[CH], b_k[CHB], b_n[CHB];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int q = tid + NT * i;
        if (TA) {
            a_k[i] = q / (BM / 4);
            a_m[i] = (q % (BM / 4)) * 4;
        } else {
            a_m[i] = q / (BK / 4);
            a_k[i] = (q % (BK / 4)) * 4;
        }
    }
#pragma unroll
    for (int i = 0; i < CHB; ++i) {
        const int q = tid + NT * i;
        if (TB) {
            b_n[i] = q / (BK / 4);
            b_k[i] = (q % (BK / 4)) * 4;
        } else {
            b_k[i] = q / (BN / 4);
            b_n[i] = (q % (BN / 4)) * 4;
        }
    }
    const float *a_ptr[CH];
    const float *b_ptr[CHB];
#pragma unroll
    for (int i = 0; i < CH; ++i)
        a_ptr[i] = TA ? A + (int64_t)a_k[i] * lda + m0 + a_m[i] : A + (int64_t)(m0 + a_m[i]) * lda + a_k[i];
#pragma unroll
    for (int i = 0; i < CHB; ++i)
        b_ptr[i] = TB ? B + (int64_t)(n0 + b_n[i]) * ldb + b_k[i] : B + (int64_t)b_k[i] * ldb + n0 + b_n[i];

    float4 ra[CH], rb[CHB];
    auto load_slab = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            ra[i] = TA ? load4_rowwise<EDGE, VEC_A>(a_ptr[i] + (int64_t)k0 * lda, K - (k0 + a_k[i]),
                                                    M - (m0 + a_m[i]))
                       : load4_rowwise<EDGE, VEC_A>(a_ptr[i] + k0, M - (m0 + a_m[i]),
                                                    K - (k0 + a_k[i]));
#pragma unroll
        for (int i = 0; i < CHB; ++i)
            rb[i] = TB ? load4_rowwise<EDGE, VEC_B>(b_ptr[i] + k0, N - (n0 + b_n[i]),
                                                    K - (k0 + b_k[i]))
                       : load4_rowwise<EDGE, VEC_B>(b_ptr[i] + (int64_t)k0 * ldb,
                                                    K - (k0 + b_k[i]), N - (n0 + b_n[i]));
    };
    // LDS images: A k-major (sm.a[k][m]) and B k-major (sm.b[k][n]) whatever the storage; a
    // chunk read along k is written as 4 scalars down a column, one read along m or n as one
    // float4 along a row.
    auto store_slab = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (TA) {
                *reinterpret_cast<float4 *>(&sm.a[buf][a_k[i]][a_m[i]]) = ra[i];
            } else {
                sm.a[buf][a_k[i] + 0][a_m[i]] = ra[i].x;
                sm.a[buf][a_k[i] + 1][a_m[i]] = ra[i].y;
                sm.a[buf][a_k[i] + 2][a_m[i]] = ra[i].z;
                sm.a[buf][a_k[i] + 3][a_m[i]] = ra[i].w;
            }
        }
#pragma unroll
        for (int i = 0; i < CHB; ++i) {
            if (TB) {
                sm.b[buf][b_k[i] + 0][b_n[i]] = rb[i].x;
                sm.b[buf][b_k[i] + 1][b_n[i]] = rb[i].y;
                sm.b[buf][b_k[i] + 2][b_n[i]] = rb[i].z;
                sm.b[buf][b_k[i] + 3][b_n[i]] = rb[i].w;
            } else {
                *reinterpret_cast<float4 *>(&sm.b[buf][b_k[i]][b_n[i]]) = rb[i];
            }
        }
    };

    float acc[TM][TN];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[m][n] = 0.0f;

    // One slab of the register-tile update from LDS stage `buf`.
    auto compute_slab = [&](int buf) {
        const float *sa = &sm.a[buf][0][0] + r0;
        const float *sb = &sm.b[buf][0][0] + c0;
        // Fragment double buffer: the reads for step k+1 are issued before the 64 FMAs of
        // step k. The scheduling barrier keeps the compiler from hoisting the whole slab's
        // reads (which would need BK*16 live registers and spill).
        float4 fa[2][MG], fb[2][NG];
#pragma unroll
        for (int g = 0; g < MG; ++g) fa[0][g] = *reinterpret_cast<const float4 *>(sa + g * 32);
#pragma unroll
        for (int g = 0; g < NG; ++g) fb[0][g] = *reinterpret_cast<const float4 *>(sb + g * 32);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const int cb = k & 1, nb = cb ^ 1;
            if (k + 1 < BK) {
#pragma unroll
                for (int g = 0; g < MG; ++g)
                    fa[nb][g] = *reinterpret_cast<const float4 *>(sa + (k + 1) * (BM + APAD) + g * 32);
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    fb[nb][g] = *reinterpret_cast<const float4 *>(sb + (k + 1) * BLD + g * 32);
                // One wait for all of step k's fragments (only step k+1's reads may still be
                // in flight; no other LDS access is outstanding inside a slab). Left to
                // itself the compiler waits fragment by fragment, and at two waves per SIMD
                // every extra instruction a wave issues is a lost FMA issue slot.
                wait_lgkmcnt<MG + NG>();
            } else {
                wait_lgkmcnt<0>();
            }
            __builtin_amdgcn_sched_barrier(0);  // no FMA is hoisted above the wait
            float ra_[TM], rb_[TN];
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                ra_[4 * g + 0] = fa[cb][g].x;
                ra_[4 * g + 1] = fa[cb][g].y;
                ra_[4 * g + 2] = fa[cb][g].z;
                ra_[4 * g + 3] = fa[cb][g].w;
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                rb_[4 * g + 0] = fb[cb][g].x;
                rb_[4 * g + 1] = fb[cb][g].y;
                rb_[4 * g + 2] = fb[cb][g].z;
                rb_[4 * g + 3] = fb[cb][g].w;
            }
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int nn = 0; nn < TN; ++nn) {
                    const int n = (F32_SNAKE && (m & 1)) ? TN - 1 - nn : nn;
                    acc[m][n] = fmaf(ra_[m], rb_[n], acc[m][n]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Software pipeline, last slab peeled. Launches without edge guards: registers hold slab
    // s+1 when slab s starts; it goes to the stage slab s-1 used (free since the last barrier)
    // before the loads of slab s+2 are issued and slab s is consumed, so the slab boundary is
    // only the barrier (each wave's stores completed long before) and the first fragment
    // reads. Measured against storing after the compute (next loop): +1.6-2.1% at 4096^3 and
    // +1.0-1.4% at 8192^3 in interleaved A/B runs on two boxes, outputs bitwise equal; with
    // the edge guards it lost up to 5% (4000^3), so edge launches keep that order. (Choosing
    // the order per tile inside an edge launch did not help either: its guarded tiles finish
    // last and set its time.)
    const int nslabs = (K + BK - 1) / BK;
    auto stage = [](int slab) { return (int)((unsigned)slab % (unsigned)ST); };
    if constexpr (ST == 1) {
        // One stage: the loads of slab s+1 are in flight while slab s is consumed; a barrier
        // frees the stage, the registers are stored, a second barrier publishes them.
        if (nslabs > 0) {
            load_slab(0);
            store_slab(0);
            __syncthreads();
            for (int s = 0; s + 1 < nslabs; ++s) {
                load_slab((s + 1) * BK);
                compute_slab(0);
                __syncthreads();
                store_slab(0);
                __syncthreads();
            }
            compute_slab(0);
        }
    } else if constexpr (F32_EARLY_STORE && !EDGE) {
        if (nslabs > 0) {
            load_slab(0);
            store_slab(0);
            if (nslabs > 1) load_slab(BK);
            __syncthreads();
            for (int s = 0; s + 1 < nslabs; ++s) {
                store_slab(stage(s + 1));
                if (s + 2 < nslabs) load_slab((s + 2) * BK);
                compute_slab(stage(s));
                // this wave's stores of slab s+1 are complete; the barrier without a fence
                // leaves the loads of slab s+2 in flight
                wait_lgkmcnt<0>();
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");
            }
            compute_slab(stage(nslabs - 1));
        }
    } else if (nslabs > 0) {
        // issue the global loads of slab s+1, consume slab s from LDS, store slab s+1 to the
        // next stage, one barrier
        load_slab(0);
        store_slab(0);
        __syncthreads();
        for (int s = 0; s + 1 < nslabs; ++s) {
            load_slab((s + 1) * BK);
            compute_slab(stage(s));
            store_slab(stage(s + 1));
            __syncthreads();
        }
        compute_slab(stage(nslabs - 1));
    }

    // Register parity of the accumulators. Each fragment quad from LDS starts at an even
    // register, so a[m] and b[n] sit in even registers for even m and n; an FMA whose three
    // registers are all even issues at two thirds of the rate. Tying each accumulator quad
    // into one register tuple with its pairs swapped puts acc[m][n] in an odd register for
    // even n, so no FMA of the loop above reads three even registers (the allocator keeps the
    // accumulators where the tuple wants them).
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            quad_t q = {acc[m][4 * h + 1], acc[m][4 * h], acc[m][4 * h + 3], acc[m][4 * h + 2]};
            asm volatile("" : "+v"(q));
            acc[m][4 * h + 1] = q[0];
            acc[m][4 * h] = q[1];
            acc[m][4 * h + 3] = q[2];
            acc[m][4 * h + 2] = q[3];
        }

    // Epilogue: rows r0 + 32*g + {0..3}, g < TM/4; columns c0 + 32*h + {0..3}, h < TN/4.
    if constexpr (!EDGE && VEC_C && TM >= 8) {
        if (beta != 0.0f) {
            // C of four rows at a time is loaded before any of their stores (element by element,
            // each load would wait for the stores before it, which may alias it; 4096^3 with
            // beta != 0 spent 10 us more than with beta = 0). (Not in the 4x4 small-tile kernel,
            // where the register allocation it leads to puts FMAs on all-odd registers.)
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                float4 old[4][NG];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                    for (int h = 0; h < NG; ++h)
                        old[mm][h] = *reinterpret_cast<const float4 *>(
                            C + (int64_t)(m0 + r0 + 32 * g + mm) * ldc + n0 + c0 + h * 32);
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const int m = 4 * g + mm;
#pragma unroll
                    for (int h = 0; h < NG; ++h)
                        *reinterpret_cast<float4 *>(C + (int64_t)(m0 + r0 + 32 * g + mm) * ldc + n0 + c0 + h * 32) =
                            make_float4(fmaf(alpha, acc[m][4 * h + 0], beta * old[mm][h].x),
                                        fmaf(alpha, acc[m][4 * h + 1], beta * old[mm][h].y),
                                        fmaf(alpha, acc[m][4 * h + 2], beta * old[mm][h].z),
                                        fmaf(alpha, acc[m][4 * h + 3], beta * old[mm][h].w));
                }
            }
            return;
        }
    }
#pragma unroll
    for (int m = 0; m < TM; ++m) {
        const int row = m0 + r0 + (m / 4) * 32 + (m % 4);
        if (EDGE && row >= M) continue;
        float *crow = C + (int64_t)row * ldc;
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            const int col = n0 + c0 + h * 32;
            float *c = crow + col;
            if (VEC_C && (!EDGE || col + 3 < N)) {
                float4 v;
                if (beta == 0.0f) {
                    v = make_float4(alpha * acc[m][4 * h + 0], alpha * acc[m][4 * h + 1],
                                    alpha * acc[m][4 * h + 2], alpha * acc[m][4 * h + 3]);
                } else {
                    const float4 old = *reinterpret_cast<const float4 *>(c);
                    v = make_float4(fmaf(alpha, acc[m][4 * h + 0], beta * old.x),
                                    fmaf(alpha, acc[m][4 * h + 1], beta * old.y),
                                    fmaf(alpha, acc[m][4 * h + 2], beta * old.z),
                                    fmaf(alpha, acc[m][4 * h + 3], beta * old.w));
                }
                *reinterpret_cast<float4 *>(c) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!EDGE || col + e < N) c[e] = epilogue_value(acc[m][4 * h + e], alpha, beta, c + e);
            }
        }
    }
}

template <class CFG, bool TA, bool TB, bool EDGE, bool VA, bool VB, bool VC>
hipError_t launch_variant(const Problem &p, hipStream_t s, int tiles_m, int tiles_n) {
    note_launch(reinterpret_cast<const void *>(&f32_regtile_kernel<CFG, TA, TB, EDGE, VA, VB, VC>), NT);
    hipLaunchKernelGGL((f32_regtile_kernel<CFG, TA, TB, EDGE, VA, VB, VC>), dim3(tiles_m * tiles_n),
                       dim3(NT), 0, s, p.M, p.N, p.K, p.alpha, (const float *)p.A, p.lda,
                       (const float *)p.B, p.ldb, p.beta, p.C, p.ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class CFG, bool EDGE, bool VA, bool VB>
hipError_t pick_c(const Problem &p, hipStream_t s, int tm, int tn, bool vc) {
    return vc ? launch_variant<CFG, false, false, EDGE, VA, VB, true>(p, s, tm, tn)
              : launch_variant<CFG, false, false, EDGE, VA, VB, false>(p, s, tm, tn);
}
template <class CFG, bool EDGE, bool VA>
hipError_t pick_b(const Problem &p, hipStream_t s, int tm, int tn, bool vb, bool vc) {
    return vb ? pick_c<CFG, EDGE, VA, true>(p, s, tm, tn, vc) : pick_c<CFG, EDGE, VA, false>(p, s, tm, tn, vc);
}
template <class CFG, bool EDGE>
hipError_t pick_a(const Problem &p, hipStream_t s, int tm, int tn, bool va, bool vb, bool vc) {
    return va ? pick_b<CFG, EDGE, true>(p, s, tm, tn, vb, vc) : pick_b<CFG, EDGE, false>(p, s, tm, tn, vb, vc);
}
// Transposed storage of A and/or B: the edge-predicated kernel unless the problem is whole
// tiles and slabs (then the unguarded one, with its earlier store order: +9% and +13% for "n t"
// and "t n" at 4096^3 in an interleaved A/B, outputs bitwise equal), vector loads and stores
// only when every operand allows them.
template <class CFG, bool TA, bool TB>
hipError_t pick_t(const Problem &p, hipStream_t s, int tm, int tn, bool edge, bool vec) {
    if (edge)
        return vec ? launch_variant<CFG, TA, TB, true, true, true, true>(p, s, tm, tn)
                   : launch_variant<CFG, TA, TB, true, false, false, false>(p, s, tm, tn);
    return vec ? launch_variant<CFG, TA, TB, false, true, true, true>(p, s, tm, tn)
               : launch_variant<CFG, TA, TB, false, false, false, false>(p, s, tm, tn);
}

// Kernel names: [edge][vec A][vec B][vec C] for row-major operands, and [layout - 1][edge][vec]
// for B stored N x K ("_nt", layout 1), A stored K x M ("_tn", 2) or both ("_tt", 3).
template <class CFG>
struct Names {
    char text[28][72];
    const char *at[2][2][2][2];
    const char *tr[3][2][2];
    Names() {
        typedef Shape<CFG::TM, CFG::TN> S;
        int n = 0;
        for (int e = 0; e < 2; ++e)
            for (int a = 0; a < 2; ++a)
                for (int b = 0; b < 2; ++b)
                    for (int c = 0; c < 2; ++c) {
                        snprintf(text[n], sizeof text[n], "f32_regtile_%dx%dx%d_%dx%d%s%s%s%s", S::BM,
                                 S::BN, CFG::BK, CFG::TM, CFG::TN, e ? "_edge" : "", a ? "_va" : "",
                                 b ? "_vb" : "", c ? "_vc" : "");
                        at[e][a][b][c] = text[n++];
                    }
        const char *lay[3] = {"_nt", "_tn", "_tt"};  // BLAS letters of op(A), op(B) storage
        for (int l = 0; l < 3; ++l)
            for (int e = 0; e < 2; ++e)
                for (int v = 0; v < 2; ++v) {
                    snprintf(text[n], sizeof text[n], "f32_regtile_%dx%dx%d_%dx%d%s%s%s", S::BM, S::BN,
                             CFG::BK, CFG::TM, CFG::TN, lay[l], e ? "_edge" : "", v ? "_vec" : "");
                    tr[l][e][v] = text[n++];
                }
    }
};

template <class CFG>
hipError_t launch_cfg(const Problem &p, hipStream_t s, const char **name) {
    typedef Shape<CFG::TM, CFG::TN> S;
    const int tiles_m = (p.M + S::BM - 1) / S::BM, tiles_n = (p.N + S::BN - 1) / S::BN;
    const bool edge = (p.M % S::BM) != 0 || (p.N % S::BN) != 0 || (p.K % CFG::BK) != 0;
    const bool va = (p.lda % 4) == 0 && aligned16(p.A);
    const bool vb = (p.ldb % 4) == 0 && aligned16(p.B);
    const bool vc = (p.ldc % 4) == 0 && aligned16(p.C);
    static const Names<CFG> names;  // thread-safe one-time initialisation
    const int layout = (p.ta ? 2 : 0) + (p.tb ? 1 : 0);
    if (layout != 0) {
        const bool vec = va && vb && vc;
        *name = names.tr[layout - 1][edge][vec];
        switch (layout) {
            case 1: return pick_t<CFG, false, true>(p, s, tiles_m, tiles_n, edge, vec);
            case 2: return pick_t<CFG, true, false>(p, s, tiles_m, tiles_n, edge, vec);
            default: return pick_t<CFG, true, true>(p, s, tiles_m, tiles_n, edge, vec);
        }
    }
    *name = names.at[edge][va][vb][vc];
    return edge ? pick_a<CFG, true>(p, s, tiles_m, tiles_n, va, vb, vc)
                : pick_a<CFG, false>(p, s, tiles_m, tiles_n, va, vb, vc);
}

}  // namespace

hipError_t launch_f32_regtile(const Problem &p, hipStream_t s, const char **name) {
    return launch_cfg<SquareCfg>(p, s, name);
}

hipError_t launch_f32_regtile_small(const Problem &p, hipStream_t s, const char **name) {
    return launch_cfg<SmallCfg>(p, s, name);
}

}  // namespace regtile
