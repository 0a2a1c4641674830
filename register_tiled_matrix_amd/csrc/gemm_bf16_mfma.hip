// gemm_bf16_mfma.hip -- rung 3 of the ladder: bf16 x bf16 -> fp32 on CDNA4 MFMA fragments.
//
// The register tile of this rung is the MFMA fragment rather than a per-thread SIMT block
// ("寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507) section 3: on CDNA the A, B and C
// fragments live in per-lane VGPRs while addresses and strides sit in SGPRs; section 3.1: the
// instruction shape sets per-lane register counts; section 3.2: each k step loads A and B
// fragments from LDS and accumulates C in place). On gfx950 (wave64) the instruction is
// v_mfma_f32_32x32x16_bf16: per lane 8 bf16 of A, 8 bf16 of B (one 16-byte LDS read each)
// and 16 fp32 accumulators; a 32x32 C block per instruction.
//
// Operands are K-contiguous on both sides (A row-major, B column-major), so A and B slabs
// share one LDS layout: a tile row (an A row, or a B column) is BK = 64 bf16 = 8 chunks of
// 16 bytes, and chunk c of row r is stored at slot c ^ key(r), key(r) = (r & 7) ^ ((r >> 3) & 1)
// (addr::slab_key for 32x32 fragments). gfx950's LDS has 64 banks and serves a 128-bit read
// 16 lanes at a time, so two addresses 256 bytes apart collide; under this key the 16 rows
// (one chunk each) of a fragment read's half-wave land in 16 distinct 16-byte bank groups,
// and the reads are free of bank conflicts (r & 7 alone left a 2-way conflict, measured).
//
// Pipeline: two LDS stages; the next slab's global loads (16-byte, coalesced: 8 lanes cover
// one 128-byte row segment) are issued into registers before the current slab's MFMAs and
// stored to the other stage after them, one barrier per slab (section 6.3's prefetch).
// Tile order: workgroups are renumbered so each XCD gets a contiguous block of tiles, walked
// in groups of 8 tile-rows (L2 reuse of A rows and B columns inside an XCD).
#include "mfma_common.h"
#include "regtile_internal.h"

namespace regtile {

namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int BK = 64;   // bf16 per slab row
constexpr int KCH = 8;   // 16-byte chunks per slab row

// Slot of 16-byte chunk `chunk` of slab row `row` (rows of 8 chunks = 128 bytes): the same
// swizzle as the DMA kernel's 32x32x16 slabs (mfma::slab_key), under which the fragment reads
// are free of LDS bank conflicts.
__device__ __forceinline__ int swz(int row, int chunk) { return row * KCH + (chunk ^ mfma::slab_key<KCH>(row)); }

// A whole run of 16 (8) bytes at any 2-byte-aligned address, as one global_load_dwordx4
// (dwordx2): the ROCm driver runs gfx9-class GPUs in unaligned-access mode, so multi-dword
// global loads take any address (the compiler emits the same single load for these copies).
__device__ __forceinline__ uint4 load16_any(const uint16_t *p) {
    uint4 r;
    __builtin_memcpy(&r, p, 16);
    return r;
}
__device__ __forceinline__ uint2 load8_any(const uint16_t *p) {
    uint2 r;
    __builtin_memcpy(&r, p, 8);
    return r;
}

template <bool EDGE, bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t *__restrict__ p, bool row_ok,
                                            int k_left) {
    // 8 consecutive bf16 starting at p (k index k0); k_left = K - k0. VEC: p is 16-byte
    // aligned; otherwise whole chunks still take one unaligned 16-byte load and only a
    // chunk cut by the end of K is read element by element.
    if (!EDGE) {
        if (VEC) return *reinterpret_cast<const uint4 *>(p);
        return load16_any(p);
    }
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0;
    if (row_ok) {
        if (k_left >= 8) return VEC ? *reinterpret_cast<const uint4 *>(p) : load16_any(p);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < k_left) v[e] = p[e];
    }
    uint4 r;
    r.x = v[0] | ((uint32_t)v[1] << 16);
    r.y = v[2] | ((uint32_t)v[3] << 16);
    r.z = v[4] | ((uint32_t)v[5] << 16);
    r.w = v[6] | ((uint32_t)v[7] << 16);
    return r;
}

// A 4 x 8 block of an operand stored K-major-outer (element (r, k) at base[k * ld + r] relative
// to the block's first element, r < 4 along the contiguous M or N dimension, k < 8), read as
// 8 runs of 4 elements along M or N and transposed in registers into 4 chunks of 8
// consecutive k, the K-contiguous form the fragment reads expect: out[j] holds row r = j,
// dword d = (k = 2d in the low half, k = 2d + 1 in the high half). The transpose is written
// out here rather than through mfma::transpose_4x8: the shared helper compiles to a
// different, measurably slower schedule in this kernel.
__device__ __forceinline__ void transpose_block(const uint32_t lo[8], const uint32_t hi[8], uint4 out[4]) {
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

// The block through a buffer descriptor over the slab's rows that lie before K (base: the
// slab's first row at the tile's first column, `rows` rows of `ld` elements), ending at the
// operand's column M - 1 (N - 1) of the last of those rows (`cols_from` = columns from the
// tile's first to the operand's last). Taken only when ld and the operand's column count are
// multiples of 4 (addr::gather_desc_takes), so that no 8-byte run crosses a row end or that
// descriptor end: rows past K read zeros, and so do the last row's columns past M or N;
// other columns past M or N read the operand's own storage and only feed outputs the
// epilogue drops. `off` is the block's byte offset from the base. Eight buffer_load_dwordx2
// with one lane offset and uniform row offsets, no predication.
__device__ __forceinline__ void load_block_mn_buf(const uint16_t *base, int64_t ld, int rows, int cols_from,
                                                  uint32_t off, uint4 out[4]) {
    const mfma::rsrc_t r = mfma::make_rsrc(base, addr::desc_bytes(rows, ld, cols_from, 2));
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const uint2 v = mfma::load_b64_buf(r, off, addr::row_run_off(kk, ld));
        lo[kk] = v.x;
        hi[kk] = v.y;
    }
    transpose_block(lo, hi, out);
}

// The block for any ld: whole runs (all 4 columns before the edge, k before K) as one
// unaligned 8-byte load, runs cut by an edge element by element; zero outside r_left x k_left.
__device__ __forceinline__ void load_block_mn_any(const uint16_t *__restrict__ p, int64_t ld, int r_left,
                                                  int k_left, uint4 out[4]) {
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const uint16_t *q = p + kk * ld;
        if (kk < k_left && r_left >= 4) {
            const uint2 v = load8_any(q);
            lo[kk] = v.x;
            hi[kk] = v.y;
        } else {
            uint32_t e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = (kk < k_left && j < r_left) ? q[j] : 0u;
            lo[kk] = e[0] | (e[1] << 16);
            hi[kk] = e[2] | (e[3] << 16);
        }
    }
    transpose_block(lo, hi, out);
}

// A_MN: A stored K x M (M-contiguous); B_MN: B stored K x N (N-contiguous). The LDS slab is
// K-contiguous either way; an MN-contiguous operand is gathered with scalar loads that are
// coalesced across lanes (consecutive lanes take consecutive M / N indices).
template <int BM, int BN, int WAVES_M, int WAVES_N, bool EDGE, bool VEC, bool VEC_C, bool F16,
          bool A_MN = false, bool B_MN = false>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void bf16_mfma_kernel(
    int M, int N, int K, float alpha, const uint16_t *__restrict__ A, int64_t lda,
    const uint16_t *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int A_CH = BM * KCH / NT;  // 16-byte chunks per thread per slab
    constexpr int B_CH = BN * KCH / NT;
    constexpr int ROWS_PER_PASS = NT / KCH;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert((BM * KCH) % NT == 0 && (BN * KCH) % NT == 0, "slab must split evenly");

    __shared__ uint4 sA[2][BM * KCH];
    __shared__ uint4 sB[2][BN * KCH];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Staging assignment: thread t owns chunk (t % KCH) of rows t / KCH + ROWS_PER_PASS * i.
    const int ld_chunk = tid % KCH;
    const int ld_row = tid / KCH;
    const uint16_t *a_src = A + (int64_t)(m0 + ld_row) * lda + ld_chunk * 8;
    const uint16_t *b_src = B + (int64_t)(n0 + ld_row) * ldb + ld_chunk * 8;
    const int64_t a_pass = (int64_t)ROWS_PER_PASS * lda;
    const int64_t b_pass = (int64_t)ROWS_PER_PASS * ldb;

    // MN-contiguous staging: thread t owns the 4 x 8 block at rows 4 (t % (B/4)), chunk
    // t / (B/4) of the slab (B = BM or BN): consecutive lanes read consecutive 8-byte runs
    // along the contiguous dimension at one k (through a descriptor when the leading
    // dimension is a multiple of 4, else as global loads with edge checks).
    static_assert(!A_MN || BM * BK == 32 * NT, "one 4 x 8 block of A per thread");
    static_assert(!B_MN || BN * BK == 32 * NT, "one 4 x 8 block of B per thread");
    const int amn_row = addr::row_block_col(tid, BM), amn_chunk = addr::row_block_kc(tid, BM);
    const int bmn_row = addr::row_block_col(tid, BN), bmn_chunk = addr::row_block_kc(tid, BN);

    uint4 ra[A_CH], rb[B_CH];
    auto load_slab = [&](int k0) {
        if (A_MN) {
            if (addr::gather_desc_takes(M, lda))
                load_block_mn_buf(A + (int64_t)k0 * lda + m0, lda, min(BK, K - k0), M - m0,
                                  addr::row_block_off(tid, BM, lda), ra);
            else
                load_block_mn_any(A + (int64_t)(k0 + amn_chunk * 8) * lda + m0 + amn_row, lda,
                                  M - (m0 + amn_row), K - (k0 + amn_chunk * 8), ra);
        } else {
#pragma unroll
            for (int i = 0; i < A_CH; ++i)
                ra[i] = load_chunk<EDGE, VEC>(a_src + i * a_pass + k0,
                                              m0 + ld_row + i * ROWS_PER_PASS < M,
                                              K - k0 - ld_chunk * 8);
        }
        if (B_MN) {
            if (addr::gather_desc_takes(N, ldb))
                load_block_mn_buf(B + (int64_t)k0 * ldb + n0, ldb, min(BK, K - k0), N - n0,
                                  addr::row_block_off(tid, BN, ldb), rb);
            else
                load_block_mn_any(B + (int64_t)(k0 + bmn_chunk * 8) * ldb + n0 + bmn_row, ldb,
                                  N - (n0 + bmn_row), K - (k0 + bmn_chunk * 8), rb);
        } else {
#pragma unroll
            for (int i = 0; i < B_CH; ++i)
                rb[i] = load_chunk<EDGE, VEC>(b_src + i * b_pass + k0,
                                              n0 + ld_row + i * ROWS_PER_PASS < N,
                                              K - k0 - ld_chunk * 8);
        }
    };
    auto store_slab = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            if (A_MN) sA[buf][swz(amn_row + i, amn_chunk)] = ra[i];
            else sA[buf][swz(ld_row + i * ROWS_PER_PASS, ld_chunk)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            if (B_MN) sB[buf][swz(bmn_row + i, bmn_chunk)] = rb[i];
            else sB[buf][swz(ld_row + i * ROWS_PER_PASS, ld_chunk)] = rb[i];
        }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Fragment rows of this lane: A rows wm*WTM + i*32 + (lane & 31); B columns likewise.
    const int frag_r = lane & 31;
    const int frag_kh = lane >> 5;  // which 8-wide half of each 16-wide k step

    auto compute_slab = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = kk * 2 + frag_kh;
            bf16x8 fa[MI], fb[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                fa[i] = __builtin_bit_cast(bf16x8, sA[buf][swz(wm * WTM + i * 32 + frag_r, chunk)]);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                fb[j] = __builtin_bit_cast(bf16x8, sB[buf][swz(wn * WTN + j * 32 + frag_r, chunk)]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = mfma::Frag<32, F16>::mfma(fa[i], fb[j], acc[i][j]);
        }
    };

    // Software pipeline with the last slab peeled (the steady-state body is one basic
    // block): global loads of slab s+1, MFMAs on slab s, LDS stores of slab s+1, barrier.
    const int nslabs = (K + BK - 1) / BK;
    if (nslabs > 0) {
        load_slab(0);
        store_slab(0);
        __syncthreads();
        for (int s = 0; s + 1 < nslabs; ++s) {
            load_slab((s + 1) * BK);
            compute_slab(s & 1);
            store_slab((s + 1) & 1);
            __syncthreads();
        }
        compute_slab((nslabs - 1) & 1);
    }

    // Epilogue. Accumulator v of lane l in a 32x32 block holds
    // row (v / 4) * 8 + (l / 32) * 4 + (v % 4), column l % 32.
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + frag_kh * 4 + (v & 3);
                if (EDGE && (row >= M || col >= N)) continue;
                float *c = C + (int64_t)row * ldc + col;
                *c = epilogue_value(acc[i][j][v], alpha, beta, c);
            }
        }
    }
    (void)VEC_C;
}

template <int BM, int BN, int WM, int WN, bool EDGE, bool VEC, bool F16, bool A_MN = false,
          bool B_MN = false>
hipError_t launch_cfg(const Problem &p, hipStream_t s) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    note_launch(reinterpret_cast<const void *>(&bf16_mfma_kernel<BM, BN, WM, WN, EDGE, VEC, false, F16, A_MN, B_MN>),
                WM * WN * 64);
    hipLaunchKernelGGL((bf16_mfma_kernel<BM, BN, WM, WN, EDGE, VEC, false, F16, A_MN, B_MN>),
                       dim3(tiles_m * tiles_n), dim3(WM * WN * 64), 0, s, p.M, p.N, p.K, p.alpha,
                       (const uint16_t *)p.A, p.lda, (const uint16_t *)p.B, p.ldb, p.beta, p.C,
                       p.ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool F16>
hipError_t launch_pick(const Problem &p, hipStream_t s, bool edge, bool vec) {
    if (edge) return vec ? launch_cfg<BM, BN, WM, WN, true, true, F16>(p, s)
                         : launch_cfg<BM, BN, WM, WN, true, false, F16>(p, s);
    return vec ? launch_cfg<BM, BN, WM, WN, false, true, F16>(p, s)
               : launch_cfg<BM, BN, WM, WN, false, false, F16>(p, s);
}

// Operands other than K-contiguous A and B: 128x128 tiles, edge-predicated kernel; `vec` only
// matters for a K-contiguous operand.
template <int BM, int BN, int WM, int WN, bool F16>
hipError_t launch_layout_tile(const Problem &p, hipStream_t s, bool vec) {
    const bool a_mn = p.ta, b_mn = !p.tb;
    if (a_mn && b_mn)
        return launch_cfg<BM, BN, WM, WN, true, false, F16, true, true>(p, s);
    if (a_mn)
        return vec ? launch_cfg<BM, BN, WM, WN, true, true, F16, true, false>(p, s)
                   : launch_cfg<BM, BN, WM, WN, true, false, F16, true, false>(p, s);
    return vec ? launch_cfg<BM, BN, WM, WN, true, true, F16, false, true>(p, s)
               : launch_cfg<BM, BN, WM, WN, true, false, F16, false, true>(p, s);
}

// 256x256 tiles of eight waves when there are enough of them to fill the chip, else 128x128.
template <bool F16>
hipError_t launch_layout(const Problem &p, hipStream_t s, bool vec, bool big) {
    return big ? launch_layout_tile<256, 256, 2, 4, F16>(p, s, vec)
               : launch_layout_tile<128, 128, 2, 2, F16>(p, s, vec);
}

#define REGTILE_STAGED_NAMES(elt, tile)                                                        \
    { elt "_mfma_" tile, elt "_mfma_" tile "_vec", elt "_mfma_" tile "_edge", elt "_mfma_" tile "_edge_vec" }
// [f16][big][edge * 2 + vec]
const char *const kStagedNames[2][2][4] = {
    {REGTILE_STAGED_NAMES("bf16", "128x128x64_w2x2"), REGTILE_STAGED_NAMES("bf16", "256x256x64_w2x4")},
    {REGTILE_STAGED_NAMES("f16", "128x128x64_w2x2"), REGTILE_STAGED_NAMES("f16", "256x256x64_w2x4")}};
#undef REGTILE_STAGED_NAMES
// [f16][big][layout code: 0 = "tt", 1 = "tn", 2 = "nn"][vec], BLAS letters of op(A), op(B)
// storage
#define REGTILE_LAYOUT_NAMES(elt, tile, lay) \
    { elt "_mfma_" tile "_" lay "_edge", elt "_mfma_" tile "_" lay "_edge_vec" }
#define REGTILE_LAYOUT_ROW(elt, tile)                                                       \
    { REGTILE_LAYOUT_NAMES(elt, tile, "tt"), REGTILE_LAYOUT_NAMES(elt, tile, "tn"),          \
      REGTILE_LAYOUT_NAMES(elt, tile, "nn") }
const char *const kLayoutNames[2][2][3][2] = {
    {REGTILE_LAYOUT_ROW("bf16", "128x128x64_w2x2"), REGTILE_LAYOUT_ROW("bf16", "256x256x64_w2x4")},
    {REGTILE_LAYOUT_ROW("f16", "128x128x64_w2x2"), REGTILE_LAYOUT_ROW("f16", "256x256x64_w2x4")}};
#undef REGTILE_LAYOUT_ROW
#undef REGTILE_LAYOUT_NAMES

}  // namespace

hipError_t launch_bf16_mfma(const Problem &p, hipStream_t s, const char **name, int shape,
                            bool f16) {
    hipError_t err = hipSuccess;
    if ((p.ta || !p.tb) && shape == 32) {
        // M/N-contiguous operands on the LDS-DMA kernel: "t n" in their own storage with
        // transposing fragment reads; "n n" / "t t" with the M/N-contiguous operand through
        // registers as rows (the transposing reads measured level or 3% slower there)
        const bool taken = p.ta == p.tb ? launch_bf16_mfma_dma_rows(p, s, name, f16, &err)
                                        : launch_bf16_mfma_dma_mn(p, s, name, f16, &err);
        if (taken) return err;
    }
    if (p.ta || !p.tb) {  // not the native K-contiguous pair
        // an M/N-contiguous operand is gathered through one descriptor per slab of 64 of its
        // rows, in 32-bit offsets: rows of 2^24 elements or more go to the naive rung
        if ((p.ta && (int64_t)BK * p.lda * 2 >= (int64_t(1) << 31)) ||
            (!p.tb && (int64_t)BK * p.ldb * 2 >= (int64_t(1) << 31)))
            return launch_bf16_naive(p, s, name, f16);
        const bool vec = (p.ta ? (p.ldb % 8) == 0 && aligned16(p.B) : (p.lda % 8) == 0 && aligned16(p.A));
        const int lay = (p.ta && p.tb) ? 0 : p.ta ? 1 : 2;  // tt: A K x M, B N x K; tn; nn
        const bool big = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) >= 256;
        *name = kLayoutNames[f16][big][lay][vec && !(p.ta && !p.tb)];
        return f16 ? launch_layout<true>(p, s, vec, big) : launch_layout<false>(p, s, vec, big);
    }
    // K a multiple of 8 and 16-byte aligned rows: the LDS-DMA kernel, else the
    // register-staged kernel below.
    if (launch_bf16_mfma_dma(p, s, name, shape, f16, &err)) return err;
    const bool vec = (p.lda % 8) == 0 && (p.ldb % 8) == 0 && aligned16(p.A) && aligned16(p.B);
    const bool big = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) >= 256;
    const int tile = big ? 256 : 128;
    const bool edge = (p.M % tile) != 0 || (p.N % tile) != 0 || (p.K % BK) != 0;
    *name = kStagedNames[f16][big][edge * 2 + vec];
    if (big)
        return f16 ? launch_pick<256, 256, 2, 4, true>(p, s, edge, vec)
                   : launch_pick<256, 256, 2, 4, false>(p, s, edge, vec);
    return f16 ? launch_pick<128, 128, 2, 2, true>(p, s, edge, vec)
               : launch_pick<128, 128, 2, 2, false>(p, s, edge, vec);
}

}  // namespace regtile
