// tile_addressing.h -- the address arithmetic of the 16-bit kernels' buffer-descriptor loads:
// where each descriptor ends, which problems each descriptor path may take, the LDS slab
// swizzle keys, and the byte offset of every lane's load. The kernels and their launchers
// compute these through the functions below, and a host-only check program enumerates every
// load of a problem's edge tiles through the same functions, so the extents are tested on the
// CPU without a GPU. Plain integer arithmetic, callable from host and device code.
//
// Operands here are row-major storage of 16-bit (or, for C, 32-bit) elements: `rows` rows of
// `ld` elements, of which the first `cols` belong to the matrix. A descriptor is based at
// element (r0, c0) of such storage. A buffer load returns zero for bytes past the descriptor's
// size (a store there is dropped), so a descriptor must end at or before the matrix's last
// element, and no load that covers a matrix element may straddle or pass its end.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define REGTILE_HD __host__ __device__ __forceinline__
#else
#define REGTILE_HD inline
#endif

namespace regtile {
namespace addr {

// Bytes of a descriptor based at (r0, c0) that spans `nrows` rows from r0 and ends at the
// last matrix element of its last row: ((nrows - 1) * ld + (cols - c0)) * esize. The caller
// passes cols_from = cols - c0 (> 0). Every byte it covers lies inside the matrix's span.
REGTILE_HD uint32_t desc_bytes(int64_t nrows, int64_t ld, int64_t cols_from, int esize) {
    return (uint32_t)(((nrows - 1) * ld + cols_from) * esize);
}

// Runs along the contiguous dimension of an M- or N-contiguous operand are `run` elements
// long and start at multiples of `run` from a tile column that is itself a multiple of `run`.
// A run never straddles a descriptor that ends at the matrix's last column when both the
// leading dimension and the column count are multiples of the run length. (16-byte DMA
// chunks: run 8; 8-byte register runs: run 4.)
REGTILE_HD bool runs_fit(int64_t cols, int64_t ld, int run) { return cols % run == 0 && ld % run == 0; }

// Swizzle of a K-contiguous slab whose rows are KCH chunks of 16 bytes: chunk c of row r sits
// in slot c ^ slab_key(r). Each key was chosen with LDS bank-conflict counters on the fragment
// read of its MFMA shape (ds_read_b128: 4.07 LDS cycles conflict-free, 8.00 for a 2-way
// conflict):
//   MF = 32 (lane l reads row l % 32 at chunk c + l / 32): (r & 7) ^ (r >> 3 & 1);
//   MF = 16 (lane l reads row l % 16 at chunk c + l / 16): (r >> 1 & 7) ^ ((r & 1) << 2).
// The second is conflict-free for both reads, the first only for MF = 32, where it measured
// 0.5% faster end to end. Both depend on r & 15 only. 64-byte rows: (r >> 2) & 3.
template <int KCH, int MF = 32>
REGTILE_HD int slab_key(int row) {
    static_assert(KCH == 4 || KCH == 8, "slab rows of 64 or 128 bytes");
    if (KCH == 8) return MF == 16 ? (((row >> 1) & 7) ^ ((row & 1) << 2)) : ((row & 7) ^ ((row >> 3) & 1));
    return (row >> 2) & 3;
}

// Swizzle of an M/N-major slab (k rows of tile-width elements): chunk c of row r at slot
// c ^ mn_key(r), spreading each half-wave's transposing reads over all 64 banks.
REGTILE_HD int mn_key(int row) { return 4 * (row & 3); }

// K-contiguous DMA (A row-major, B stored N x K): slot p = (wave * J + j) * 64 + lane of a
// stage holds chunk (p % KCH) ^ key(row) of tile row p / KCH. Lane part of instruction j's
// byte offset (rows and chunk of instruction j & 1; the uniform part adds the rest).
template <int KCH, int MF>
REGTILE_HD uint32_t kc_dma_lane(int wave, int J, int j, int lane, int64_t ld, int *chunk_k) {
    const int p = (wave * J + j) * 64 + lane;
    const int r = p / KCH, c = (p % KCH) ^ slab_key<KCH, MF>(r);
    *chunk_k = c * 8;  // first k of the chunk within the slab
    return (uint32_t)(r * ld + c * 8) * 2u;
}
// Uniform part of DMA instruction q of the slab starting at k0 (instruction q's rows are
// instruction (q & 1)'s plus (q & ~1) * 64 / KCH).
template <int KCH>
REGTILE_HD uint32_t kc_dma_instr(int q, int k0, int64_t ld) {
    return (uint32_t)(q & ~1) * (uint32_t)((64 / KCH) * ld) * 2u + (uint32_t)k0 * 2u;
}
// Chunks of the last slab that lie past K take this bit: the offset then passes every tile
// descriptor's end (each spans less than 2^31 bytes) and the chunk loads as zeros.
constexpr uint32_t kPastEnd = 0x80000000u;

// M/N-major DMA ("t n"): a slab of 64 k-rows of MCH = tile width / 8 chunks; one instruction
// covers MROWS = 64 / MCH rows. Lane part of instruction j (the key repeats every two
// instructions: J is even and MROWS is 2 or 4), and the uniform part of instruction q of a
// wave's J for the slab at k0.
REGTILE_HD uint32_t mn_dma_lane(int lane, int j, int64_t ld, int mch) {
    const int mrows = 64 / mch;
    const int r_in = lane / mch, slot = lane % mch, key = mn_key(mrows * j + r_in);
    return (uint32_t)(r_in * ld + (slot ^ key) * 8) * 2u;
}
REGTILE_HD uint32_t mn_dma_instr(int wave, int J, int q, int k0, int64_t ld, int mch) {
    return (uint32_t)((64 / mch) * (wave * J + q) + k0) * (uint32_t)ld * 2u;
}

// 4 x 8 blocks of an M/N-contiguous operand read as 8-byte runs (the register-row path of the
// DMA kernel and the gather of the register-staged kernel): block b of a slab of `width`
// columns sits at column 4 (b % (width / 4)), k chunk b / (width / 4). Lane byte offset of the
// block from the slab base; run kk adds kk * ld * 2 (and the slab's k0 * ld * 2 where the
// descriptor is based at row 0).
REGTILE_HD int row_block_col(int b, int width) { return (b % (width / 4)) * 4; }
REGTILE_HD int row_block_kc(int b, int width) { return b / (width / 4); }
REGTILE_HD uint32_t row_block_off(int b, int width, int64_t ld) {
    return (uint32_t)((row_block_kc(b, width) * 8) * ld + row_block_col(b, width)) * 2u;
}
REGTILE_HD uint32_t row_run_off(int k, int64_t ld) { return (uint32_t)k * (uint32_t)ld * 2u; }

// The split-K kernel (gemm_bf16_mfma_splitk.hip) stages 64x64 tiles. A K-contiguous operand
// takes the K-contiguous DMA layout above (kc_dma_lane / kc_dma_instr, 64-row tiles, four
// waves). An M/N-contiguous one keeps its storage: a slab of 64 k-rows of 8 chunks (the tile's
// 64 columns), chunk c of row r at slot c ^ sk_mn_key(r); DMA instruction q of wave w fills
// rows 8 (2 w + q) .. + 7, lane l row l / 8 of those at slot l % 8 (mn_dma_instr with 8
// chunks per row gives the uniform part). A transposing fragment read takes 4 consecutive rows
// and 4 chunks in each 32 lanes; rows two apart lie 256 bytes apart, on the same banks, so the
// key moves the chunks of every other pair of rows to the row's other 64 bytes, and the 32
// lanes reach 256 distinct bytes. It depends on row bit 1 only, so every instruction's lanes
// share it.
REGTILE_HD int sk_mn_key(int row) { return 4 * ((row >> 1) & 1); }
REGTILE_HD uint32_t sk_mn_dma_lane(int lane, int64_t ld) {
    const int r_in = lane >> 3, slot = lane & 7;
    return (uint32_t)(r_in * ld + (slot ^ sk_mn_key(r_in)) * 8) * 2u;
}
// Problems it takes, in storage order (ta: A stored K x M; tb: B stored N x K, the 16-bit
// native form). A K-contiguous operand: K a multiple of 8 (every chunk lies wholly before or
// wholly past K), leading dimension a multiple of 8 and 64 rows within 2^30 bytes, so that a
// lane offset carrying kPastEnd plus any uniform part stays below 2^32. An M/N-contiguous
// operand: column count and leading dimension multiples of 8 (no chunk straddles the
// descriptor's end) and K + 64 rows within 2^31 bytes.
REGTILE_HD bool sk_dma_takes(bool ta, bool tb, int M, int N, int K, int64_t lda, int64_t ldb) {
    const int64_t lim30 = int64_t(1) << 30, lim31 = int64_t(1) << 31;
    auto kc_ok = [&](int64_t ld) { return K % 8 == 0 && ld % 8 == 0 && 64 * ld * 2 < lim30; };
    auto mn_ok = [&](int64_t cols, int64_t ld) { return runs_fit(cols, ld, 8) && ((int64_t)K + 64) * ld * 2 + 512 < lim31; };
    return K > 0 && (ta ? mn_ok(M, lda) : kc_ok(lda)) && (tb ? kc_ok(ldb) : mn_ok(N, ldb));
}

// C fragment layout of the two gfx950 MFMA shapes: accumulator v of lane l of an MF x MF
// block sits at row c_row_lane(l) + c_row_acc(v), column l % MF.
//   MF = 32 (32x32x16): row (l / 32) * 4 + (v / 4) * 8 + v % 4;
//   MF = 16 (16x16x32): row (l / 16) * 4 + v.
template <int MF>
REGTILE_HD int c_row_lane(int lane) { return MF == 32 ? (lane >> 5) * 4 : (lane >> 4) * 4; }
template <int MF>
REGTILE_HD constexpr int c_row_acc(int v) { return MF == 32 ? (v >> 2) * 8 + (v & 3) : v; }

// Epilogue byte offsets into a C descriptor based at the tile's first element: a lane part
// (the wave's place in the tile and the lane's fragment row and column) and a uniform part
// per fragment (i, j) and accumulator v. Lanes whose column lies at or past N take kPastEnd
// instead of the lane part, so their stores pass the descriptor's end and are dropped.
template <int MF>
REGTILE_HD uint32_t c_lane_off(int row0, int col0, int lane, int64_t ldc) {
    return (uint32_t)((row0 + c_row_lane<MF>(lane)) * ldc + col0 + lane % MF) * 4u;
}
template <int MF>
REGTILE_HD uint32_t c_acc_off(int i, int j, int v, int64_t ldc) {
    return (uint32_t)((i * MF + c_row_acc<MF>(v)) * ldc + j * MF) * 4u;
}

// Which problems the DMA kernel's descriptor paths take (the launchers add the pointer
// alignment: 16 bytes for a DMA operand, 8 for a row operand). Tile edge: 256, or 128 when
// the problem has at most 128 tiles of 256x256. Every descriptor and every uniform offset
// added to kPastEnd stays below 2^31 bytes.
REGTILE_HD int dma_tile(int M, int N) {
    return (int64_t)((M + 255) / 256) * ((N + 255) / 256) <= 128 ? 128 : 256;
}
// both operands K-contiguous (A row-major, B stored N x K)
REGTILE_HD bool kc_dma_takes(int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
    const int64_t t = dma_tile(M, N), lim = int64_t(1) << 31;
    return K > 0 && K % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && t * lda * 2 < lim &&
           t * ldb * 2 < lim && t * ldc * 4 < lim;
}
// "t n": A stored K x M and B stored K x N, both in their own storage (16-byte chunks)
REGTILE_HD bool mn_dma_takes(int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
    const int64_t t = dma_tile(M, N), lim = int64_t(1) << 31;
    return K > 0 && runs_fit(M, lda, 8) && runs_fit(N, ldb, 8) && ((int64_t)K + 64) * lda * 2 + 512 < lim &&
           ((int64_t)K + 64) * ldb * 2 + 512 < lim && t * ldc * 4 < lim;
}
// "n n" (B stored K x N is the row operand) or "t t" (A stored K x M is): the other operand
// K-contiguous over DMA, the row operand as 8-byte runs
REGTILE_HD bool rows_dma_takes(bool nn, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
    const int64_t t = dma_tile(M, N), lim = int64_t(1) << 31;
    const int64_t ld_dma = nn ? lda : ldb, ld_row = nn ? ldb : lda;
    const int64_t cols_row = nn ? N : M;
    return K > 0 && K % 8 == 0 && ld_dma % 8 == 0 && t * ld_dma * 2 < lim && runs_fit(cols_row, ld_row, 4) &&
           ((int64_t)K + 128) * ld_row * 2 + 512 < lim && t * ldc * 4 < lim;
}
// The register-staged kernel's gather of an M/N-contiguous operand with `cols` columns goes
// through a per-slab descriptor (8-byte runs) when this holds, else through predicated loads.
REGTILE_HD bool gather_desc_takes(int64_t cols, int64_t ld) { return runs_fit(cols, ld, 4); }

}  // namespace addr
}  // namespace regtile
