// extent_check.cpp -- host replay of the 16-bit MFMA kernels' buffer-descriptor accesses.
//
// For one problem and one operand arrangement, every load and store that the edge tiles of the
// LDS-DMA kernel (and the register-staged kernel's M/N-contiguous gather) issue through a buffer
// descriptor is enumerated on the CPU. Each byte offset comes from the same functions the
// kernels call (register_tiled_matrix_amd/csrc/tile_addressing.h); this file only repeats the
// loops over waves, lanes, instructions and slabs. For every problem the launchers would take,
// it checks that
//   1. every descriptor lies inside the span of the matrix it covers (first to last element),
//   2. every load that covers a matrix element lies wholly inside its descriptor (a load that
//      straddles or passes the end reads zeros, so a matrix element there would be lost),
//   3. no load or store offset wraps past 2^32,
//   4. every matrix element of a tile's slab is loaded exactly once inside the descriptor,
//   5. every store inside the C descriptor writes an element of C, each element of the tile
//      exactly once.
// Usage:
//   extent_check one <kc|tn|nn|tt|gather|sk|sk_tn|sk_nn|sk_tt> M N K lda ldb ldc
//   extent_check force ...                   (the same, also where the launcher would refuse)
//   extent_check sweep <seed> <count>        (seeded shapes the launchers take, every path)
// Prints one line per violation (at most 20) and a summary; exit status 1 on any violation.
// Built with -DEXTENT_LOOSE it checks the earlier descriptor sizes (K full rows of the M/N-
// contiguous operand), which must fail: the check's own control.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <string>
#include <vector>

#include "tile_addressing.h"

namespace {

using namespace regtile;

long g_violations = 0, g_loads = 0, g_stores = 0;
bool g_force = false;  // enumerate even problems the launchers would not take (controls)

void violation(const char *what, const std::string &ctx) {
    if (g_violations < 20) std::printf("VIOLATION %s: %s\n", what, ctx.c_str());
    ++g_violations;
}

// Row-major storage of a matrix: `rows` rows of `ld` elements, the first `cols` of each real.
struct Mat {
    int64_t rows, cols, ld;
    int esize;
    int64_t span() const { return (rows - 1) * ld + cols; }  // elements from first to last
    bool real(int64_t idx) const { return idx >= 0 && idx / ld < rows && idx % ld < cols; }
};

// A descriptor based at element `base` of a matrix, `bytes` long.
struct Desc {
    int64_t base;
    uint64_t bytes;
};

void check_desc(const Mat &m, const Desc &d, const std::string &ctx) {
    if (d.base < 0 || d.base + (int64_t)(d.bytes / m.esize) > m.span() || d.bytes % m.esize != 0)
        violation("descriptor outside the matrix", ctx);
}

std::string fmt(const char *f, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, f);
    std::vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    return buf;
}

// Coverage of one tile slab: nr x nc positions (r0 + i, c0 + j) of a matrix.
struct Cover {
    int64_t r0, c0, nr, nc;
    std::vector<uint8_t> n;
    Cover(int64_t r0_, int64_t c0_, int64_t nr_, int64_t nc_) : r0(r0_), c0(c0_), nr(nr_), nc(nc_), n(nr_ * nc_, 0) {}
    bool in(int64_t r, int64_t c) const { return r >= r0 && r < r0 + nr && c >= c0 && c < c0 + nc; }
    void hit(int64_t r, int64_t c) { ++n[(r - r0) * nc + (c - c0)]; }
    void verify(const Mat &m, const std::string &ctx) {
        for (int64_t i = 0; i < nr; ++i)
            for (int64_t j = 0; j < nc; ++j) {
                const int64_t r = r0 + i, c = c0 + j;
                if (r < m.rows && c < m.cols && n[i * nc + j] != 1) {
                    violation("matrix element of the tile not covered exactly once",
                              ctx + fmt(" at (%ld, %ld) x%d", (long)r, (long)c, (int)n[i * nc + j]));
                    return;
                }
            }
    }
};

// One access of `len` elements at byte offset voff + soff from the descriptor base, meant for
// the elements (row, col) .. (row, col + len - 1) of the matrix (the position the kernel's
// layout assigns it, derived here independently of the offset functions). Checks that the
// offset addresses that position (unless it carries kPastEnd), that it does not wrap, that an
// access meant for any matrix element lies wholly inside the descriptor, and that a store
// inside the descriptor is meant for matrix elements only. Counts the matrix elements it
// delivers into `cov`.
void access(const Mat &m, const Desc &d, uint32_t voff, uint32_t soff, int len, bool store, int64_t row,
            int64_t col, Cover *cov, const std::string &ctx) {
    const uint64_t off = (uint64_t)voff + soff;
    (store ? g_stores : g_loads)++;
    if (off >= (uint64_t(1) << 32)) {
        violation("offset wraps past 2^32", ctx);
        return;
    }
    const bool flagged = (voff & addr::kPastEnd) != 0;
    if (!flagged && d.base + (int64_t)(off / m.esize) != row * m.ld + col)
        violation("offset does not address the element the layout assigns", ctx);
    const bool inside = off + (uint64_t)len * m.esize <= d.bytes;
    int n_real = 0;
    for (int u = 0; u < len; ++u) n_real += row < m.rows && col + u < m.cols;
    if (n_real > 0 && !inside)
        violation(off < d.bytes ? "access straddles the descriptor end over a matrix element"
                                : "access past the descriptor end is meant for a matrix element",
                  ctx);
    if (store && inside && n_real < len) violation("store inside the descriptor to a non-matrix element", ctx);
    if (store && !inside && off < d.bytes) violation("store straddles the descriptor end", ctx);
    if (inside && cov)
        for (int u = 0; u < len; ++u)
            if (row < m.rows && col + u < m.cols) {
                if (cov->in(row, col + u))
                    cov->hit(row, col + u);
                else
                    violation("access meant for an element outside its tile slab", ctx);
            }
}

constexpr int BK = 64, KCH = 8, NWAVES = 4;

// The slabs worth enumerating: all when few, else the first two and the last two, plus the
// clamped repeat of the last that the pipeline issues past the end.
std::vector<int> slabs_of(int nslabs) {
    std::vector<int> s;
    if (nslabs <= 8) {
        for (int i = 0; i < nslabs; ++i) s.push_back(i);
    } else {
        s = {0, 1, nslabs - 2, nslabs - 1};
    }
    s.push_back(nslabs);  // clamped to the last slab
    return s;
}
std::vector<int64_t> tiles_of(int64_t extent, int64_t t) {
    const int64_t n = (extent + t - 1) / t;
    std::vector<int64_t> v{0};
    if (n > 2) v.push_back((n - 2) * t);
    if (n > 1) v.push_back((n - 1) * t);
    return v;
}

// K-contiguous operand over DMA: `rows` (M or N) rows of K elements at leading dimension ld.
// Layout: slot p = (wave * J + q) * 64 + lane of a stage holds tile row p / 8, chunk
// (p % 8) ^ slab_key(row) (8 elements of k); chunks of the last slab past K are flagged.
// past_zero: loads for slabs past the last take offsets flagged past the end (zeros, meant for
// no element), as the split-K kernel issues them; otherwise they repeat the last slab.
template <int MF>
void check_kc_operand(const char *name, int64_t rows, int K, int64_t ld, int t, bool past_zero = false) {
    const Mat m{rows, K, ld, 2};
    const bool ktail = K % BK != 0;
    const int nslabs = ktail ? (K + BK - 1) / BK : K / BK, k_last = (nslabs - 1) * BK;
    const int J = t * KCH / (64 * NWAVES);
    for (int64_t r0 : tiles_of(rows, t)) {
        const int64_t nrows = std::min<int64_t>(t, rows - r0);
        const Desc d{r0 * ld, addr::desc_bytes(nrows, ld, K, 2)};
        const std::string head = fmt("kc %s MF %d tile %ld rows %ld K %d ld %ld", name, MF, (long)r0, (long)rows, K, (long)ld);
        check_desc(m, d, head);
        for (int s : slabs_of(nslabs)) {
            const int k0 = std::min(s, nslabs - 1) * BK;
            Cover cov(r0, k0, t, BK);
            for (int w = 0; w < NWAVES; ++w)
                for (int q = 0; q < J; ++q)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int p = (w * J + q) * 64 + lane, r = p / KCH;
                        const bool past = past_zero && s >= nslabs;
                        const int64_t col = (past ? (int64_t)nslabs * BK : k0) + 8 * ((p % KCH) ^ addr::slab_key<KCH, MF>(r));
                        int ck;
                        uint32_t voff = addr::kc_dma_lane<KCH, MF>(w, J, q & 1, lane, ld, &ck);
                        if (past || (ktail && k0 == k_last && k_last + ck >= K)) voff |= addr::kPastEnd;
                        access(m, d, voff, addr::kc_dma_instr<KCH>(q, k0, ld), 8, false, r0 + r, col,
                               s < nslabs ? &cov : nullptr, head + fmt(" slab %d wave %d instr %d lane %d", s, w, q, lane));
                    }
            if (s < nslabs) cov.verify(m, head + fmt(" slab %d", s));
        }
    }
}

// M/N-major operand of the split-K kernel: K rows of `cols` (M or N) elements at ld, 64-wide
// tiles. A slab is 64 k-rows of 8 chunks; instruction q of wave w fills rows 8 (2 w + q) ..,
// lane l row l / 8 of those, slot l % 8, holding chunk slot ^ sk_mn_key(row). Slabs past the
// last load zeros (offsets flagged past the end).
void check_sk_mn_operand(const char *name, int64_t cols, int K, int64_t ld) {
    const Mat m{K, cols, ld, 2};
    const int nslabs = (K + BK - 1) / BK;
    for (int64_t c0 : tiles_of(cols, 64)) {
        const std::string head = fmt("sk-mn %s tile col %ld cols %ld K %d ld %ld", name, (long)c0, (long)cols, K, (long)ld);
        const Desc d{c0, addr::desc_bytes(K, ld, cols - c0, 2)};
        check_desc(m, d, head);
        for (int s : slabs_of(nslabs)) {
            const int k0 = std::min(s, nslabs - 1) * BK;
            Cover cov(k0, c0, BK, 64);
            for (int w = 0; w < NWAVES; ++w)
                for (int q = 0; q < 2; ++q)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int row = 8 * (2 * w + q) + lane / 8;  // within the slab
                        const int64_t col = c0 + 8 * ((lane % 8) ^ addr::sk_mn_key(row));
                        const bool past = s >= nslabs;  // meant for no element: rows from K on
                        uint32_t voff = addr::sk_mn_dma_lane(lane, ld);
                        if (past) voff |= addr::kPastEnd;
                        access(m, d, voff, addr::mn_dma_instr(w, 2, q, k0, ld, 8), 8, false,
                               (past ? (int64_t)nslabs * BK : k0) + row, col,
                               s < nslabs ? &cov : nullptr, head + fmt(" slab %d wave %d instr %d lane %d", s, w, q, lane));
                    }
            if (s < nslabs) cov.verify(m, head + fmt(" slab %d", s));
        }
    }
}

// M/N-major operand over DMA ("t n"): K rows of `cols` (M or N) elements at ld. Layout: a slab
// is 64 k-rows of t / 8 chunks; instruction q of wave w fills rows 64 / (t/8) * (w J + q) ..,
// lane l row l / (t/8) of those, slot l % (t/8), holding chunk slot ^ mn_key(row).
void check_mn_operand(const char *name, int64_t cols, int K, int64_t ld, int t) {
    const Mat m{K, cols, ld, 2};
    const int nslabs = (K + BK - 1) / BK;
    const int mch = t / 8, mrows = 64 / mch, J = t * KCH / (64 * NWAVES);
    for (int64_t c0 : tiles_of(cols, t)) {
        const std::string head = fmt("tn %s tile col %ld cols %ld K %d ld %ld", name, (long)c0, (long)cols, K, (long)ld);
#ifdef EXTENT_LOOSE
        const Desc d{c0, (uint64_t)K * ld * 2};
#else
        const Desc d{c0, addr::desc_bytes(K, ld, cols - c0, 2)};
#endif
        check_desc(m, d, head);
        for (int s : slabs_of(nslabs)) {
            const int k0 = std::min(s, nslabs - 1) * BK;
            Cover cov(k0, c0, BK, t);
            for (int w = 0; w < NWAVES; ++w)
                for (int q = 0; q < J; ++q)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int row = mrows * (w * J + q) + lane / mch;  // within the slab
                        const int64_t col = c0 + 8 * ((lane % mch) ^ addr::mn_key(row));
                        access(m, d, addr::mn_dma_lane(lane, q & 1, ld, mch), addr::mn_dma_instr(w, J, q, k0, ld, mch), 8,
                               false, k0 + row, col, s < nslabs ? &cov : nullptr,
                               head + fmt(" slab %d wave %d instr %d lane %d", s, w, q, lane));
                    }
            if (s < nslabs) cov.verify(m, head + fmt(" slab %d", s));
        }
    }
}

// Row operand of "n n" / "t t": K rows of `cols` elements at ld, 8-byte runs through registers.
// Layout: block b of a slab (width t) covers columns 4 (b % (t/4)) .. +3 at k rows
// 8 (b / (t/4)) .. +7; thread tid owns blocks tid + 256 i.
void check_row_operand(const char *name, int64_t cols, int K, int64_t ld, int t) {
    const Mat m{K, cols, ld, 2};
    const bool ktail = K % BK != 0;
    const int nslabs = ktail ? (K + BK - 1) / BK : K / BK;
    const int NT = NWAVES * 64, blocks = (t / 4) * KCH / NT;
    for (int64_t c0 : tiles_of(cols, t)) {
        const std::string head = fmt("rows %s tile col %ld cols %ld K %d ld %ld", name, (long)c0, (long)cols, K, (long)ld);
#ifdef EXTENT_LOOSE
        const Desc d{c0, (uint64_t)K * ld * 2};
#else
        const Desc d{c0, addr::desc_bytes(K, ld, cols - c0, 2)};
#endif
        check_desc(m, d, head);
        for (int s : slabs_of(nslabs + 1)) {  // the pipeline loads up to slab nslabs + 1, clamped
            const int k0 = std::min(s, nslabs - 1) * BK;
            Cover cov(k0, c0, BK, t);
            for (int tid = 0; tid < NT; ++tid)
                for (int i = 0; i < blocks; ++i)
                    for (int kk = 0; kk < 8; ++kk) {
                        const int b = tid + NT * i;
                        const int64_t col = c0 + 4 * (b % (t / 4)), k = k0 + 8 * (b / (t / 4)) + kk;
                        access(m, d, addr::row_block_off(b, t, ld), addr::row_run_off(k0 + kk, ld), 4, false, k, col,
                               s < nslabs ? &cov : nullptr, head + fmt(" slab %d thread %d block %d run %d", s, tid, i, kk));
                    }
            if (s < nslabs) cov.verify(m, head + fmt(" slab %d", s));
        }
    }
}

// The register-staged kernel's gather of an M/N-contiguous operand through one descriptor per
// slab (taken when addr::gather_desc_takes): K rows of `cols` at ld, tile width t, nt threads
// (one 4 x 8 block each, as in the row operand).
void check_gather_operand(const char *name, int64_t cols, int K, int64_t ld, int t, int nt) {
    const Mat m{K, cols, ld, 2};
    const int nslabs = (K + BK - 1) / BK;
    for (int64_t c0 : tiles_of(cols, t)) {
        for (int s : slabs_of(nslabs)) {
            if (s == nslabs) continue;  // this kernel issues no clamped repeat
            const int k0 = s * BK, rows = std::min(BK, K - k0);
            const std::string head =
                fmt("gather %s tile %d col %ld slab %d cols %ld K %d ld %ld", name, t, (long)c0, s, (long)cols, K, (long)ld);
#ifdef EXTENT_LOOSE
            const Desc d{k0 * ld + c0, (uint64_t)rows * ld * 2};
#else
            const Desc d{k0 * ld + c0, addr::desc_bytes(rows, ld, cols - c0, 2)};
#endif
            check_desc(m, d, head);
            Cover cov(k0, c0, BK, t);
            for (int tid = 0; tid < nt; ++tid)
                for (int kk = 0; kk < 8; ++kk) {
                    const int64_t col = c0 + 4 * (tid % (t / 4)), k = k0 + 8 * (tid / (t / 4)) + kk;
                    access(m, d, addr::row_block_off(tid, t, ld), addr::row_run_off(kk, ld), 4, false, k, col, &cov,
                           head + fmt(" thread %d run %d", tid, kk));
                }
            cov.verify(m, head);
        }
    }
}

// The DMA kernel's epilogue: C (M x N at ldc, fp32) through a descriptor per tile. Layout:
// 2 x 2 waves of t/2 x t/2; fragment (i, j) of a wave is an MF x MF block; accumulator v of
// lane l sits at row (l / 32) 4 + (v / 4) 8 + v % 4 (MF 32) or (l / 16) 4 + v (MF 16), column
// l % MF.
template <int MF>
void check_c(int M, int N, int64_t ldc, int t) {
    const Mat m{M, N, ldc, 4};
    const int wtm = t / 2, wtn = t / 2, MI = wtm / MF, NI = wtn / MF, NACC = MF * MF / 64;
    for (int64_t m0 : tiles_of(M, t))
        for (int64_t n0 : tiles_of(N, t)) {
            const std::string head = fmt("C MF %d tile (%ld, %ld) M %d N %d ldc %ld", MF, (long)m0, (long)n0, M, N, (long)ldc);
            const Desc d{m0 * ldc + n0, addr::desc_bytes(std::min<int64_t>(t, M - m0), ldc, N - n0, 4)};
            check_desc(m, d, head);
            Cover cov(m0, n0, t, t);
            for (int w = 0; w < NWAVES; ++w) {
                const int wm = w / 2, wn = w % 2;
                for (int lane = 0; lane < 64; ++lane)
                    for (int j = 0; j < NI; ++j) {
                        const int64_t col = n0 + wn * wtn + j * MF + lane % MF;
                        const uint32_t lo = col < N ? addr::c_lane_off<MF>(wm * wtm, wn * wtn, lane, ldc) : addr::kPastEnd;
                        for (int i = 0; i < MI; ++i)
                            for (int v = 0; v < NACC; ++v) {
                                const int in_frag = MF == 32 ? (lane / 32) * 4 + (v / 4) * 8 + v % 4 : (lane / 16) * 4 + v;
                                const int64_t row = m0 + wm * wtm + i * MF + in_frag;
                                access(m, d, lo, addr::c_acc_off<MF>(i, j, v, ldc), 1, true, row, col, &cov,
                                       head + fmt(" wave %d lane %d frag %d acc %d", w, lane, i * NI + j, v));
                            }
                    }
            }
            cov.verify(m, head);
        }
}

// Every descriptor access one arrangement makes for one problem (if its launcher takes it).
// Returns false when the launcher would not take the problem.
bool check_problem(const std::string &path, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
    const int t = addr::dma_tile(M, N);
    if (path == "kc") {
        if (!addr::kc_dma_takes(M, N, K, lda, ldb, ldc) && !g_force) return false;
        if (t == 256) {  // 256x256 tiles run either fragment shape; 128x128 only 32x32x16
            check_kc_operand<16>("A", M, K, lda, t);
            check_kc_operand<16>("B", N, K, ldb, t);
            check_c<16>(M, N, ldc, t);
        }
        check_kc_operand<32>("A", M, K, lda, t);
        check_kc_operand<32>("B", N, K, ldb, t);
        check_c<32>(M, N, ldc, t);
        return true;
    }
    if (path.rfind("sk", 0) == 0) {  // split-K kernel, 64x64 tiles: sk ("n t"), sk_tn, sk_nn, sk_tt
        const bool ta = path == "sk_tn" || path == "sk_tt", tb = path == "sk" || path == "sk_tt";
        if (!addr::sk_dma_takes(ta, tb, M, N, K, lda, ldb) && !g_force) return false;
        if (ta) check_sk_mn_operand("A", M, K, lda);
        else check_kc_operand<32>("A", M, K, lda, 64, true);
        if (tb) check_kc_operand<32>("B", N, K, ldb, 64, true);
        else check_sk_mn_operand("B", N, K, ldb);
        return true;
    }
    if (path == "tn") {
        if (!addr::mn_dma_takes(M, N, K, lda, ldb, ldc) && !g_force) return false;
        check_mn_operand("A", M, K, lda, t);
        check_mn_operand("B", N, K, ldb, t);
        check_c<32>(M, N, ldc, t);
        return true;
    }
    if (path == "nn" || path == "tt") {
        const bool nn = path == "nn";
        if (!addr::rows_dma_takes(nn, M, N, K, lda, ldb, ldc) && !g_force) return false;
        if (nn) {
            check_kc_operand<32>("A", M, K, lda, t);
            check_row_operand("B", N, K, ldb, t);
        } else {
            check_row_operand("A", M, K, lda, t);
            check_kc_operand<32>("B", N, K, ldb, t);
        }
        check_c<32>(M, N, ldc, t);
        return true;
    }
    if (path == "gather") {  // A stored K x M (lda), B stored K x N (ldb), both tile sizes
        bool any = false;
        for (int tile : {128, 256}) {
            const int nt = tile == 256 ? 512 : 256;
            if (addr::gather_desc_takes(M, lda) || g_force) check_gather_operand("A", M, K, lda, tile, nt), any = true;
            if (addr::gather_desc_takes(N, ldb) || g_force) check_gather_operand("B", N, K, ldb, tile, nt), any = true;
        }
        return any;
    }
    std::fprintf(stderr, "unknown path %s\n", path.c_str());
    std::exit(2);
}

}  // namespace

int main(int argc, char **argv) {
    if (argc == 9 && (std::strcmp(argv[1], "one") == 0 || std::strcmp(argv[1], "force") == 0)) {
        g_force = std::strcmp(argv[1], "force") == 0;
        const bool taken = check_problem(argv[2], std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                                         std::atoll(argv[6]), std::atoll(argv[7]), std::atoll(argv[8]));
        std::printf("%s loads %ld stores %ld violations %ld\n", taken ? "taken" : "not-taken", g_loads, g_stores,
                    g_violations);
        return g_violations ? 1 : 0;
    }
    if (argc == 4 && std::strcmp(argv[1], "sweep") == 0) {
        std::mt19937_64 rng(std::strtoull(argv[2], nullptr, 10));
        const int count = std::atoi(argv[3]);
        // edge-heavy sizes: 1, tiny, around the tile sizes and the slab depth, primes
        const int sizes[] = {1, 2, 3, 4, 7, 8, 12, 16, 24, 56, 63, 64, 65, 96, 120, 127, 128, 129, 136, 200,
                             248, 255, 256, 257, 263, 264, 384, 509, 512, 520, 1000, 1088, 1504, 2040};
        const int n_sizes = sizeof sizes / sizeof sizes[0];
        const char *paths[] = {"kc", "tn", "nn", "tt", "gather", "sk", "sk_tn", "sk_nn", "sk_tt"};
        long taken = 0;
        for (int c = 0; c < count; ++c) {
            const int M = sizes[rng() % n_sizes], N = sizes[rng() % n_sizes], K = sizes[rng() % n_sizes];
            for (const char *path : paths) {
                // leading dimensions: the smallest legal, or that plus a small pad
                const std::string p = path;
                const bool a_km = p == "tn" || p == "tt" || p == "gather" || p == "sk_tn" || p == "sk_tt";
                const bool b_kn = p == "tn" || p == "nn" || p == "gather" || p == "sk_tn" || p == "sk_nn";
                const int64_t lda = (a_km ? M : K) + (rng() % 3 == 0 ? 8 * (int64_t)(rng() % 3) : 0);
                const int64_t ldb = (b_kn ? N : K) + (rng() % 3 == 0 ? 8 * (int64_t)(rng() % 3) : 0);
                const int64_t ldc = N + (rng() % 3 == 0 ? (int64_t)(rng() % 5) : 0);
                taken += check_problem(p, M, N, K, lda, ldb, ldc);
            }
        }
        std::printf("sweep problems-taken %ld loads %ld stores %ld violations %ld\n", taken, g_loads, g_stores,
                    g_violations);
        return g_violations ? 1 : 0;
    }
    std::fprintf(stderr, "usage: extent_check one <kc|tn|nn|tt|gather|sk|sk_tn|sk_nn|sk_tt> M N K lda ldb ldc | sweep <seed> <count>\n");
    return 2;
}
