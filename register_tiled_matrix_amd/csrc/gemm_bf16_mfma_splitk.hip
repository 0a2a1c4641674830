// gemm_bf16_mfma_splitk.hip -- the bf16 / fp16 MFMA kernel for problems with few output tiles:
// K split over the waves of a workgroup.
//
// 1024 x 1024 has 64 tiles of 128x128, so the LDS-DMA kernel (gemm_bf16_mfma_dma.hip) keeps a
// quarter of the 256 CUs busy however deep K is. Here a workgroup owns a 64x64 tile (256 of them
// for 1024 x 1024), and each of its 4 waves accumulates that whole tile, as 2 x 2 fragments of
// 32x32 (64 fp32 accumulators per lane), over its own share of K: wave w takes 16-wide k step w
// of every 64-deep slab ("寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507) section 3.2: per
// k step the A and B fragments come from LDS into VGPRs and the C accumulators are updated in
// place; sections 2.4 and 7.2: tile size traded against the number of resident waves). The four
// partial tiles are summed through LDS in a fixed order, so the results are deterministic.
//
// Slabs reach LDS by LDS DMA (buffer_load_dwordx4 ... lds through per-tile buffer descriptors)
// in the LDS-DMA kernel's K-contiguous layout: 128-byte slab rows, so each DMA instruction covers
// eight whole rows (tile_addressing.h, kc_dma_lane / kc_dma_instr with 64-row tiles: each wave
// loads 16 rows of A and 16 of B per slab). The ring holds R slabs. In iteration s a wave
//   * waits for its fragments of slab s (read in iteration s - 1) and reads those of slab s + 1;
//   * issues its four MFMAs of slab s, each followed by one of its DMA loads of slab s + R - 1
//     into the slot that slab s - 1 left (free since the barrier that ended iteration s - 1);
//   * waits for its own loads of slab s + 2 and meets the other waves at the barrier, which
//     publishes slab s + 2 and frees slab s's slot.
// The MFMAs are in the pipe while the wave waits at the barrier, and the fragments the next
// iteration's MFMAs use were read an iteration earlier. A slab's loads have R - 3 iterations to
// land. Loads for slabs past the last read zeros without touching memory (offsets past the
// descriptors' ends), so every iteration waits on the same counts.
//
// Edges: each tile's descriptors end at the matrix's last element, so rows past M (columns past
// N) load zeros; in the K tail the chunks of the last slab past K take an offset past the
// descriptor's end and load zeros too. C is written with plain stores, guarded by row and column.
#include <type_traits>

#include "mfma_common.h"
#include "regtile_internal.h"

namespace regtile {

namespace {
using namespace mfma;

constexpr int SK_T = 64;                  // tile edge
constexpr int SK_BK = 64;                 // slab depth
constexpr int SK_KCH = SK_BK / 8;         // 16-byte chunks per slab row
constexpr int SK_NW = 4;                  // waves: one 16-wide k step of each slab apiece
constexpr int SK_J = SK_T * SK_KCH / (64 * SK_NW);  // DMA instructions per operand, wave and slab
constexpr int SK_OP = SK_T * SK_KCH;      // 16-byte slots of one operand in a slab
constexpr int SK_SLAB = 2 * SK_OP;        // A then B: 16 KB
constexpr int SK_PSTRIDE = SK_T + 8;      // row stride (floats) of a partial tile in LDS
constexpr int SK_NT = SK_NW * 64;
constexpr int SK_TPR = SK_NT / SK_T;      // epilogue threads per row
constexpr int SK_SW = SK_T / SK_TPR;      // columns per epilogue thread
static_assert(SK_J == 2 && SK_SW % 4 == 0, "two DMA instructions per operand; whole float4 strips");

// MN: bit 0, A is stored K x M; bit 1, B is stored K x N (M/N-major slabs, transposing reads).
template <int R, bool F16, bool KTAIL, int MN>
__global__ __launch_bounds__(SK_NT) void bf16_mfma_splitk_kernel(
    int M, int N, int K, float alpha, const uint16_t *__restrict__ A, int64_t lda,
    const uint16_t *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int vec_c) {
    constexpr int MF = 32;
    typedef Frag<MF, F16> F;
    constexpr int MI = SK_T / MF, NI = SK_T / MF;
    constexpr int SLOTS_RING = R * SK_SLAB, SLOTS_PART = SK_NW * SK_T * SK_PSTRIDE / 4;
    static_assert(R >= 4 && 4 * (R - 2) < 64, "ring of at least four slabs; vmcnt range");
    static_assert(SLOTS_RING * 16 <= 160 * 1024 && SLOTS_PART <= SLOTS_RING, "LDS");
    constexpr bool A_MN = (MN & 1) != 0, B_MN = (MN & 2) != 0;
    static_assert(!(KTAIL && MN == 3), "the K tail of M/N-major operands is the descriptors' end");
    __shared__ uint4 smem[SLOTS_RING];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * SK_T, n0 = tn * SK_T;

    // Descriptors: over the tile's rows of a K-contiguous operand, ending at element K - 1 of its
    // last real row; over the K rows of an M/N-major operand from the tile's first column,
    // ending at the operand's last element (rows past K, and that row's columns past M or N,
    // load zeros; other columns past M or N only feed outputs that are never stored).
    const rsrc_t a_rsrc = A_MN ? make_rsrc(A + m0, addr::desc_bytes(K, lda, M - m0, 2))
                               : make_rsrc(A + (int64_t)m0 * lda, addr::desc_bytes(min(SK_T, M - m0), lda, K, 2));
    const rsrc_t b_rsrc = B_MN ? make_rsrc(B + n0, addr::desc_bytes(K, ldb, N - n0, 2))
                               : make_rsrc(B + (int64_t)n0 * ldb, addr::desc_bytes(min(SK_T, N - n0), ldb, K, 2));
    const int nslabs = (K + SK_BK - 1) / SK_BK;
    const int k_last = (nslabs - 1) * SK_BK;
    uint32_t a_voff[SK_J], b_voff[SK_J], a_voff_last[SK_J], b_voff_last[SK_J];
#pragma unroll
    for (int j = 0; j < SK_J; ++j) {
        int ka, kb;  // first k of each lane's chunk within the slab
        a_voff[j] = addr::kc_dma_lane<SK_KCH, MF>(wave, SK_J, j, lane, lda, &ka);
        b_voff[j] = addr::kc_dma_lane<SK_KCH, MF>(wave, SK_J, j, lane, ldb, &kb);
        a_voff_last[j] = k_last + ka < K ? a_voff[j] : a_voff[j] | addr::kPastEnd;
        b_voff_last[j] = k_last + kb < K ? b_voff[j] : b_voff[j] | addr::kPastEnd;
        if (A_MN) a_voff[j] = a_voff_last[j] = addr::sk_mn_dma_lane(lane, lda);
        if (B_MN) b_voff[j] = b_voff_last[j] = addr::sk_mn_dma_lane(lane, ldb);
    }
    auto soff_a = [&](int q, int k0) {
        return A_MN ? addr::mn_dma_instr(wave, SK_J, q, k0, lda, SK_KCH) : addr::kc_dma_instr<SK_KCH>(q, k0, lda);
    };
    auto soff_b = [&](int q, int k0) {
        return B_MN ? addr::mn_dma_instr(wave, SK_J, q, k0, ldb, SK_KCH) : addr::kc_dma_instr<SK_KCH>(q, k0, ldb);
    };
    // DMA instruction d (0, 1: A; 2, 3: B) of this wave for slab `slab` into ring slot `slot`.
    // A slab past the last takes offsets past the descriptors' ends: it fills its (unused)
    // slot with zeros without touching memory, and keeps every wait's count the same.
    auto dma_one = [&](int slab, int slot, int d) {
        const bool past = slab >= nslabs;
        const int k0 = min(slab, nslabs - 1) * SK_BK;
        const bool last = KTAIL && k0 == k_last;
        const int q = d & 1;
        uint4 *dst = smem + slot * SK_SLAB + (d >> 1) * SK_OP + (wave * SK_J + q) * 64;
        const uint32_t va = past ? a_voff[q] | addr::kPastEnd : last ? a_voff_last[q] : a_voff[q];
        const uint32_t vb = past ? b_voff[q] | addr::kPastEnd : last ? b_voff_last[q] : b_voff[q];
        if (d < 2)
            dma16_buf(a_rsrc, va, soff_a(q, k0), dst);
        else
            dma16_buf(b_rsrc, vb, soff_b(q, k0), dst);
    };

    typename F::acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < F::NACC; ++v) acc[i][j][v] = 0.0f;

    // Fragment reads of this wave's k step (chunks 2 w and 2 w + 1 of each row) of the slab in
    // ring slot `slot` into register buffer `buf`: lane l reads row 32 i + l % 32 (A) or column
    // 32 j + l % 32 (B) at chunk 2 w + l / 32, conflict-free under the slab key.
    const int frag_r = lane & 31, chunk = 2 * wave + (lane >> 5);
    // M/N-major fragment (two ds_read_b64_tr_b16): in each group of 16 lanes, lane t addresses
    // k row 16 w + 8 (l / 32) + t / 4 (+ 4 for the second read) at columns 16 ((l / 16) % 2) +
    // 4 (t % 4) .. + 3 of the fragment, so that lane l receives column l % 32 at the 8 k of its
    // group (mfma_common.h states the transposing read's lane mapping). Rows r and r + 4 share
    // the key.
    const int tr_t = lane & 15;
    const int tr_row = 16 * wave + 8 * (lane >> 5) + (tr_t >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_t & 3);
    auto mn_frag = [&](const uint4 *part, int col0) {
        const char *base = reinterpret_cast<const char *>(part);
        const int col = col0 + tr_col;
        const int off = ((col >> 3) ^ addr::sk_mn_key(tr_row)) * 16 + (col & 7) * 2;
        const uint2 lo = lds_read_tr16(base + tr_row * (SK_KCH * 16) + off);
        const uint2 hi = lds_read_tr16(base + (tr_row + 4) * (SK_KCH * 16) + off);
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    bf16x8 fa[2][MI], fb[2][NI];
    auto read_frags = [&](int slot, int buf) {
        const uint4 *sa = smem + slot * SK_SLAB, *sb = sa + SK_OP;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if constexpr (A_MN) {
                fa[buf][i] = mn_frag(sa, i * MF);
            } else {
                const int row = i * MF + frag_r;
                fa[buf][i] = __builtin_bit_cast(bf16x8, sa[row * SK_KCH + (chunk ^ slab_key<SK_KCH, MF>(row))]);
            }
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if constexpr (B_MN) {
                fb[buf][j] = mn_frag(sb, j * MF);
            } else {
                const int row = j * MF + frag_r;
                fb[buf][j] = __builtin_bit_cast(bf16x8, sb[row * SK_KCH + (chunk ^ slab_key<SK_KCH, MF>(row))]);
            }
        }
    };
    constexpr int NREAD = MI * (A_MN ? 2 : 1) + NI * (B_MN ? 2 : 1);  // LDS reads per k step
    auto wrap = [](int x) { return x >= R ? x - R : x; };

    // iteration s on register buffer CB (compile-time, so the buffers stay in registers);
    // `slot` is slab s's ring slot
    auto iteration = [&](int s, int slot, auto cb_tag) {
        constexpr int CB = decltype(cb_tag)::value;
        wait_lgkmcnt0();  // slab s's fragments are in registers
        __builtin_amdgcn_sched_barrier(0);
        read_frags(wrap(slot + 1), CB ^ 1);  // slab s + 1, published a barrier ago
        const int refill = wrap(slot + R - 1);  // slab s - 1's slot
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                const int j = (i & 1) ? NI - 1 - jj : jj;  // consecutive MFMAs share an operand
                acc[i][j] = F::mfma(fa[CB][i], fb[CB][j], acc[i][j]);
            }
#pragma unroll
        for (int d = 0; d < 4; ++d) dma_one(s + R - 1, refill, d);
        // order: the fragment reads, then MFMA and DMA load in turn
        __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<4 * (R - 3)>();  // own loads of slab s + 2 have landed
        lds_barrier();              // slab s + 2 published; slab s's slot read by nobody any more
    };

    // prologue: slabs 0 .. R - 2 into slots 0 .. R - 2; slab 0's fragments; slab 1 published
#pragma unroll
    for (int s = 0; s + 1 < R; ++s)
#pragma unroll
        for (int d = 0; d < 4; ++d) dma_one(s, s, d);
    wait_vmcnt<4 * (R - 2)>();  // own loads of slab 0
    lds_barrier();
    read_frags(0, 0);
    wait_vmcnt<4 * (R - 3)>();  // own loads of slab 1
    lds_barrier();
    int slot = 0;
    for (int s = 0; s < nslabs; s += 2) {
        iteration(s, slot, std::integral_constant<int, 0>{});
        slot = wrap(slot + 1);
        if (s + 1 < nslabs) {
            iteration(s + 1, slot, std::integral_constant<int, 1>{});
            slot = wrap(slot + 1);
        }
    }
    wait_vmcnt<0>();  // no DMA may still be writing the ring when it turns into partial tiles

    // The epilogue's strip of C (beta != 0) is read before the reduction, so that its latency
    // overlaps the partial-tile exchange: thread t owns row t / TPR, columns (t % TPR) SW ..
    // + SW - 1 of the tile.
    constexpr int SW = SK_SW, TPR = SK_TPR;
    const int erow = tid / TPR, ecol = (tid % TPR) * SW;
    const int grow = m0 + erow;
    float4 cold[SW / 4];
    const bool row_ok = grow < M;
    if (beta != 0.0f && row_ok) {
        const float *crow = C + (int64_t)grow * ldc + n0 + ecol;
#pragma unroll
        for (int c4 = 0; c4 < SW / 4; ++c4) {
            const int gcol = n0 + ecol + 4 * c4;
            if (vec_c && gcol + 3 < N) {
                cold[c4] = *reinterpret_cast<const float4 *>(crow + 4 * c4);
            } else {
                float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (gcol + u < N) e[u] = crow[4 * c4 + u];
                cold[c4] = make_float4(e[0], e[1], e[2], e[3]);
            }
        }
    }
    __syncthreads();  // every wave is done with the ring

    // Partial tile of wave w at rows of SK_PSTRIDE floats (the two half-waves of a store, 4
    // rows apart, land on different banks); accumulator v of fragment (i, j) of lane l is
    // element (32 i + row_lane(l) + row_acc(v), 32 j + l % 32).
    float *part = reinterpret_cast<float *>(smem);
    {
        float *mine = part + wave * SK_T * SK_PSTRIDE;
        const int rl = F::row_lane(lane), cl = lane % MF;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v)
                    mine[(i * MF + rl + F::row_acc(v)) * SK_PSTRIDE + j * MF + cl] = acc[i][j][v];
    }
    __syncthreads();

    // Sum of the four partials in wave order, then the epilogue.
    if (!row_ok) return;
    float *crow = C + (int64_t)grow * ldc + n0 + ecol;
#pragma unroll
    for (int c4 = 0; c4 < SW / 4; ++c4) {
        const int col = ecol + 4 * c4, gcol = n0 + col;
        float4 s = *reinterpret_cast<const float4 *>(&part[erow * SK_PSTRIDE + col]);
#pragma unroll
        for (int w = 1; w < SK_NW; ++w) {
            const float4 p = *reinterpret_cast<const float4 *>(&part[(w * SK_T + erow) * SK_PSTRIDE + col]);
            s.x += p.x;
            s.y += p.y;
            s.z += p.z;
            s.w += p.w;
        }
        float4 v;
        if (beta == 0.0f) {  // C is never read
            v = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
        } else {
            const float4 o = cold[c4];
            v = make_float4(fmaf(alpha, s.x, beta * o.x), fmaf(alpha, s.y, beta * o.y),
                            fmaf(alpha, s.z, beta * o.z), fmaf(alpha, s.w, beta * o.w));
        }
        if (vec_c && gcol + 3 < N) {
            *reinterpret_cast<float4 *>(crow + 4 * c4) = v;
        } else {
            const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (gcol + u < N) crow[4 * c4 + u] = sv[u];
        }
    }
}

// ring of R slabs (16 KB each)
#ifndef SK_RING
#define SK_RING 8
#endif

template <bool F16, bool KTAIL, int MN>
hipError_t launch_sk(const Problem &p, hipStream_t s) {
    const int tiles_m = (p.M + SK_T - 1) / SK_T, tiles_n = (p.N + SK_T - 1) / SK_T;
    const int vec_c = (p.ldc % 4) == 0 && aligned16(p.C);
    note_launch(reinterpret_cast<const void *>(&bf16_mfma_splitk_kernel<SK_RING, F16, KTAIL, MN>), SK_NT);
    hipLaunchKernelGGL((bf16_mfma_splitk_kernel<SK_RING, F16, KTAIL, MN>), dim3(tiles_m * tiles_n), dim3(SK_NT), 0,
                       s, p.M, p.N, p.K, p.alpha, (const uint16_t *)p.A, p.lda, (const uint16_t *)p.B, p.ldb,
                       p.beta, p.C, p.ldc, tiles_m, tiles_n, vec_c);
    return hipGetLastError();
}
template <bool F16, int MN>
hipError_t launch_sk_tail(const Problem &p, hipStream_t s, bool ktail) {
    if constexpr (MN == 3)
        return launch_sk<F16, false, 3>(p, s);
    else
        return ktail ? launch_sk<F16, true, MN>(p, s) : launch_sk<F16, false, MN>(p, s);
}
template <bool F16>
hipError_t launch_sk_layout(const Problem &p, hipStream_t s, int mn, bool ktail) {
    switch (mn) {
        case 1: return launch_sk_tail<F16, 1>(p, s, ktail);
        case 2: return launch_sk_tail<F16, 2>(p, s, ktail);
        case 3: return launch_sk_tail<F16, 3>(p, s, ktail);
        default: return launch_sk_tail<F16, 0>(p, s, ktail);
    }
}

}  // namespace

// Takes (and launches, status in *err) a problem whose operands meet addr::sk_dma_takes in
// their storage: A row-major or stored K x M, B stored N x K (the native form) or K x N,
// 16-byte aligned; returns false, launching nothing, otherwise. M, N and K may end anywhere.
bool launch_bf16_mfma_splitk(const Problem &p, hipStream_t s, const char **name, bool f16, hipError_t *err) {
    if (!addr::sk_dma_takes(p.ta, p.tb, p.M, p.N, p.K, p.lda, p.ldb) || !aligned16(p.A) || !aligned16(p.B))
        return false;
    const int mn = (p.ta ? 1 : 0) | (p.tb ? 0 : 2);
    const bool ktail = mn != 3 && p.K % SK_BK != 0;  // a K-contiguous operand's last slab
#define REGTILE_SK_NAME(elt, lay) elt "_mfma32x32x16_splitk4_64x64x64" lay
#define REGTILE_SK_PAIR(elt, lay) {REGTILE_SK_NAME(elt, lay), REGTILE_SK_NAME(elt, lay) "_ktail"}
#define REGTILE_SK_SET(elt) \
    {REGTILE_SK_PAIR(elt, ""), REGTILE_SK_PAIR(elt, "_tt"), REGTILE_SK_PAIR(elt, "_nn"), REGTILE_SK_PAIR(elt, "_tn")}
    // [f16][mn: 0 "n t" (native), 1 "t t", 2 "n n", 3 "t n"][ktail]
    static const char *const names[2][4][2] = {REGTILE_SK_SET("bf16"), REGTILE_SK_SET("f16")};
#undef REGTILE_SK_SET
#undef REGTILE_SK_PAIR
#undef REGTILE_SK_NAME
    *name = names[f16][mn][ktail];
    *err = f16 ? launch_sk_layout<true>(p, s, mn, ktail) : launch_sk_layout<false>(p, s, mn, ktail);
    return true;
}

}  // namespace regtile
