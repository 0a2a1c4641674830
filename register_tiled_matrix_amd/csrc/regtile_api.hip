// regtile_api.hip -- the C ABI declared in include/regtile.h: argument validation (before any
// HIP call), the BLAS quick returns, the kernel-ladder selector and launch on the caller's
// stream. The library never allocates, frees or synchronises.
#include "regtile.h"

#include <math.h>

#include "regtile_internal.h"

namespace {

thread_local const char *g_last_kernel = "none";
thread_local const void *g_last_fn = nullptr;  // the kernel behind g_last_kernel, if one ran
thread_local unsigned g_last_threads = 0;

// LAPACK-style validation. `shift` counts the arguments before M (1 for the *_algo entry
// points, 3 for the *_ex ones), so the returned -i always names the position in the called
// function. ta / tb select the leading-dimension rules of transposed storage (A stored K x M:
// lda >= M; B stored N x K: ldb >= K).
int validate(int shift, int M, int N, int K, float alpha, const void *A, int lda, const void *B,
             int ldb, float *C, int ldc, bool ta, bool tb) {
    if (M < 0) return -(1 + shift);
    if (N < 0) return -(2 + shift);
    if (K < 0) return -(3 + shift);
    const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    if (reads_ab && A == nullptr) return -(5 + shift);
    const int lda_min = ta ? M : K;
    if (lda < (lda_min > 1 ? lda_min : 1)) return -(6 + shift);
    if (reads_ab && B == nullptr) return -(7 + shift);
    const int ldb_min = tb ? K : N;
    if (ldb < (ldb_min > 1 ? ldb_min : 1)) return -(8 + shift);
    if (M > 0 && N > 0 && C == nullptr) return -(10 + shift);
    if (ldc < (N > 1 ? N : 1)) return -(11 + shift);
    return REGTILE_OK;
}

int finish(hipError_t err, const char *name) {
    g_last_kernel = name;
    return err == hipSuccess ? REGTILE_OK : (int)err;
}

regtile::Problem make_problem(int M, int N, int K, float alpha, const void *A, int lda,
                              const void *B, int ldb, float beta, float *C, int ldc, bool ta,
                              bool tb) {
    regtile::Problem p;
    p.ta = ta;
    p.tb = tb;
    p.M = M;
    p.N = N;
    p.K = K;
    p.alpha = alpha;
    p.beta = beta;
    p.A = A;
    p.lda = lda;
    p.B = B;
    p.ldb = ldb;
    p.C = C;
    p.ldc = ldc;
    return p;
}

// Quick returns shared by both element types. Returns true when the call is complete. Every
// path that launches first clears any error left pending by an earlier, unrelated runtime
// call, which would otherwise be reported as this launch's status; M == 0 or N == 0 makes no
// HIP call at all.
bool quick_return(const regtile::Problem &p, hipStream_t s, int *status) {
    if (p.M == 0 || p.N == 0) {
        g_last_kernel = "quick-return";
        g_last_fn = nullptr;
        *status = REGTILE_OK;
        return true;
    }
    (void)hipGetLastError();
    if (p.K == 0 || p.alpha == 0.0f) {
        const char *name = "scale_c";
        *status = finish(regtile::launch_scale_c(p, s, &name), name);
        return true;
    }
    return false;
}

bool bad_flag(int f) { return f != 0 && f != 1; }

int run_f32(int shift, int algo, bool ta, bool tb, int M, int N, int K, float alpha,
            const float *A, int lda, const float *B, int ldb, float beta, float *C, int ldc,
            void *stream) {
    if (algo < REGTILE_F32_AUTO || algo > REGTILE_F32_REGTILE_SMALL) return -1;
    // the LDS-tiled and split-K rungs stage row-major operands only
    if ((ta || tb) && (algo == REGTILE_F32_LDS || algo == REGTILE_F32_SPLITK)) return -1;
    const int v = validate(shift, M, N, K, alpha, A, lda, B, ldb, C, ldc, ta, tb);
    if (v != REGTILE_OK) return v;
    const regtile::Problem p = make_problem(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ta, tb);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int status;
    if (quick_return(p, s, &status)) return status;
    const char *name = "none";
    hipError_t err;
    if (algo == REGTILE_F32_AUTO) {
        // The square kernel (128x256 tiles, two workgroups = two waves per SIMD per CU) needs
        // about 1.5 tiles per CU: with 256 tiles (one per CU, one wave per SIMD) it ran at
        // 66 TFLOP/s on 4096x2048x4096 against 86 for split-K, with 384 it led (93 against 87).
        // Below that, smaller tiles restore the parallelism: the split-K kernel for row-major
        // operands once K is long enough to pay for its reduction (K >= 1024, or K >= 384
        // while fewer than four 64x64 tiles per CU leave the small-tile kernel under-filled),
        // otherwise 64x64 tiles of 4x4 micro-tiles at 4 waves per SIMD (bitwise equal to the
        // naive rung). Measured on 30 shapes with 64 <= K <= 8192. Problems of fewer than 448
        // such tiles take split-K from K >= 128 (eight waves on each 64x64 tile, or 32x32 tiles
        // below 64 of them from K >= 64): at 1024x1024x256 40.3 against 30.5 TFLOP/s.
        const int64_t sq = (int64_t)((M + 127) / 128) * ((N + 255) / 256);
        const int64_t tiles64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
        if (sq >= 384)
            algo = REGTILE_F32_REGTILE;
        else if (!ta && !tb && (K >= 1024 || (tiles64 < 4 * 256 && K >= 384) || (tiles64 < 448 && K >= 128) ||
                                (tiles64 < 64 && K >= 64)))
            algo = REGTILE_F32_SPLITK;
        else
            algo = REGTILE_F32_REGTILE_SMALL;
    }
    switch (algo) {
        case REGTILE_F32_NAIVE: err = regtile::launch_f32_naive(p, s, &name); break;
        case REGTILE_F32_LDS: err = regtile::launch_f32_lds(p, s, &name); break;
        case REGTILE_F32_SPLITK: err = regtile::launch_f32_splitk(p, s, &name); break;
        case REGTILE_F32_REGTILE_SMALL: err = regtile::launch_f32_regtile_small(p, s, &name); break;
        default: err = regtile::launch_f32_regtile(p, s, &name); break;
    }
    return finish(err, name);
}

int run_16b(bool f16, int shift, int algo, bool ta, bool tb, int M, int N, int K, float alpha,
            const uint16_t *A, int lda, const uint16_t *B, int ldb, float beta, float *C, int ldc,
            void *stream) {
    if (algo < REGTILE_BF16_AUTO || algo > REGTILE_BF16_MFMA_SPLITK) return -1;
    const int v = validate(shift, M, N, K, alpha, A, lda, B, ldb, C, ldc, ta, tb);
    if (v != REGTILE_OK) return v;
    const regtile::Problem p = make_problem(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ta, tb);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int status;
    if (quick_return(p, s, &status)) return status;
    const char *name = "none";
    hipError_t err;
    switch (algo) {
        case REGTILE_BF16_AUTO:
            if (!(regtile::bf16_splitk_preferred(p) && regtile::launch_bf16_mfma_splitk(p, s, &name, f16, &err)))
                err = regtile::launch_bf16_mfma(p, s, &name, 32, f16);
            break;
        case REGTILE_BF16_NAIVE: err = regtile::launch_bf16_naive(p, s, &name, f16); break;
        case REGTILE_BF16_MFMA_16X16: err = regtile::launch_bf16_mfma(p, s, &name, 16, f16); break;
        case REGTILE_BF16_MFMA_SPLITK:
            if (!regtile::launch_bf16_mfma_splitk(p, s, &name, f16, &err))
                err = regtile::launch_bf16_mfma(p, s, &name, 32, f16);
            break;
        default: err = regtile::launch_bf16_mfma(p, s, &name, 32, f16); break;
    }
    return finish(err, name);
}

}  // namespace

namespace regtile {
void note_launch(const void *kernel, unsigned threads) {
    g_last_fn = kernel;
    g_last_threads = threads;
}
}  // namespace regtile

extern "C" {

int gemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream) {
    return run_f32(0, REGTILE_F32_AUTO, false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   stream);
}

int gemm_bf16(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
              int ldb, float beta, float *C, int ldc, void *stream) {
    return run_16b(false, 0, REGTILE_BF16_AUTO, false, true, M, N, K, alpha, A, lda, B, ldb, beta,
                   C, ldc, stream);
}

int regtile_gemm_f32_algo(int algo, int M, int N, int K, float alpha, const float *A, int lda,
                          const float *B, int ldb, float beta, float *C, int ldc, void *stream) {
    return run_f32(1, algo, false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int regtile_gemm_bf16_algo(int algo, int M, int N, int K, float alpha, const uint16_t *A,
                           int lda, const uint16_t *B, int ldb, float beta, float *C, int ldc,
                           void *stream) {
    return run_16b(false, 1, algo, false, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
             int ldb, float beta, float *C, int ldc, void *stream) {
    return run_16b(true, 0, REGTILE_BF16_AUTO, false, true, M, N, K, alpha, A, lda, B, ldb, beta,
                   C, ldc, stream);
}

int regtile_gemm_f16_algo(int algo, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                          const uint16_t *B, int ldb, float beta, float *C, int ldc, void *stream) {
    return run_16b(true, 1, algo, false, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int regtile_gemm_f32_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb, float beta, float *C,
                        int ldc, void *stream) {
    if (bad_flag(trans_a)) return -2;
    if (bad_flag(trans_b)) return -3;
    return run_f32(3, algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int regtile_gemm_bf16_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                         const uint16_t *A, int lda, const uint16_t *B, int ldb, float beta,
                         float *C, int ldc, void *stream) {
    if (bad_flag(trans_a)) return -2;
    if (bad_flag(trans_b)) return -3;
    return run_16b(false, 3, algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   stream);
}

int regtile_gemm_f16_ex(int algo, int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const uint16_t *A, int lda, const uint16_t *B, int ldb, float beta,
                        float *C, int ldc, void *stream) {
    if (bad_flag(trans_a)) return -2;
    if (bad_flag(trans_b)) return -3;
    return run_16b(true, 3, algo, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   stream);
}

const char *regtile_last_kernel(void) { return g_last_kernel; }

int regtile_last_kernel_info(regtile_kernel_info *info) {
    if (info == nullptr) return -1;
    *info = regtile_kernel_info{};
    if (g_last_fn == nullptr) return (int)hipErrorInvalidDeviceFunction;
    hipFuncAttributes a;
    hipError_t e = hipFuncGetAttributes(&a, g_last_fn);
    if (e != hipSuccess) return (int)e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g_last_fn, (int)g_last_threads, 0);
    if (e != hipSuccess) return (int)e;
    info->workgroup_size = (int)g_last_threads;
    info->registers = a.numRegs;
    info->lds_bytes = (int)a.sharedSizeBytes;
    info->scratch_bytes = (int)a.localSizeBytes;
    info->workgroups_per_cu = per_cu;
    info->waves_per_simd = per_cu * (int)((g_last_threads + 63) / 64) / 4;
    return REGTILE_OK;
}

const char *regtile_strerror(int status) {
    if (status == REGTILE_OK) return "success";
    if (status < 0) {
        static thread_local char buf[96];
        snprintf(buf, sizeof buf, "invalid argument at position %d", -status);
        return buf;
    }
    return hipGetErrorString(static_cast<hipError_t>(status));
}

int regtile_version(void) { return 100; }

}  // extern "C"
