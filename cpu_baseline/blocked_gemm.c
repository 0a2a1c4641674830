/*
 * blocked_gemm.c -- blocked, multithreaded fp32 CPU GEMM used as a performance baseline.
 *
 * BENCHMARK BASELINE ONLY: timed by bench.py next to the GPU kernels; the product (the HIP
 * library) never calls it, and it is not the correctness reference (that is oracle/).
 *
 * C = alpha * A * B + beta * C, row-major A (M x K, lda), B (K x N, ldb), C (M x N, ldc),
 * fp32 storage and fp32 accumulation.
 *
 * Structure: the register micro-tile is the CPU-SIMD form of register tiling described in
 * "寄存器Tiling跨架构解析" (www.zskr.cn/news/2170507), sections 5.1-5.2: an 8 x 16 fp32 tile of C
 * held in vector registers (8 rows x two 8-wide vectors), updated per k by broadcasting one
 * element of A and multiplying with a 16-wide row slice of B. Around it sit cache blocks
 * (KC x NC panels of B packed once per block, MC x KC panels of A packed per thread) and an
 * OpenMP loop over row blocks. Vector code uses GCC vector extensions sized for AVX2 (8 floats);
 * build with -O3 -mavx2 -mfma.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef float v8f __attribute__((vector_size(32)));

enum { MR = 8, NR = 16, MC = 128, KC = 256, NC = 2048 };

int blocked_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Pack a KC x NC block of B (rows k0.., columns j0..) into NR-wide column strips,
 * zero-padding past n. Layout: strip s, then k, then NR values. */
static void pack_b(int kc, int nc, const float *B, long ldb, float *Bp)
{
    for (int s = 0; s < (nc + NR - 1) / NR; ++s) {
        const int j0 = s * NR, w = nc - j0 < NR ? nc - j0 : NR;
        float *dst = Bp + (long)s * kc * NR;
        for (int k = 0; k < kc; ++k) {
            const float *src = B + (long)k * ldb + j0;
            int j = 0;
            for (; j < w; ++j) dst[k * NR + j] = src[j];
            for (; j < NR; ++j) dst[k * NR + j] = 0.0f;
        }
    }
}

/* Pack an MC x KC block of A into MR-tall row strips (strip, k, MR values), zero-padded. */
static void pack_a(int mc, int kc, const float *A, long lda, float *Ap)
{
    for (int s = 0; s < (mc + MR - 1) / MR; ++s) {
        const int i0 = s * MR, h = mc - i0 < MR ? mc - i0 : MR;
        float *dst = Ap + (long)s * kc * MR;
        for (int k = 0; k < kc; ++k) {
            int i = 0;
            for (; i < h; ++i) dst[k * MR + i] = A[(long)(i0 + i) * lda + k];
            for (; i < MR; ++i) dst[k * MR + i] = 0.0f;
        }
    }
}

/* 8 x 16 register tile: acc[r][0..1] += a[r] * b[0..15] for each k, then
 * C[r][c] += alpha * acc[r][c] for the h x w part of the tile inside C. */
static void micro_kernel(int kc, const float *Ap, const float *Bp, float alpha, float *C, long ldc,
                         int h, int w)
{
    v8f acc[MR][2];
    for (int r = 0; r < MR; ++r)
        acc[r][0] = acc[r][1] = (v8f){0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < kc; ++k) {
        v8f b0, b1;
        memcpy(&b0, Bp + k * NR, sizeof b0);
        memcpy(&b1, Bp + k * NR + 8, sizeof b1);
        const float *a = Ap + k * MR;
        for (int r = 0; r < MR; ++r) {
            const v8f ar = (v8f){a[r], a[r], a[r], a[r], a[r], a[r], a[r], a[r]};
            acc[r][0] += ar * b0;
            acc[r][1] += ar * b1;
        }
    }
    float t[MR][NR];
    memcpy(t, acc, sizeof t);
    for (int r = 0; r < h; ++r)
        for (int c = 0; c < w; ++c)
            C[r * ldc + c] += alpha * t[r][c];
}

int blocked_sgemm(long M, long N, long K, float alpha, const float *A, long lda, const float *B,
                  long ldb, float beta, float *C, long ldc)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i)
        for (long j = 0; j < N; ++j)
            C[i * ldc + j] = beta == 0.0f ? 0.0f : beta * C[i * ldc + j];
    if (K == 0 || alpha == 0.0f)
        return 0;
    float *Bp = (float *)aligned_alloc(64, sizeof(float) * (size_t)KC * ((NC + NR - 1) / NR) * NR);
    if (!Bp)
        return -2;
    int status = 0;
    for (long j0 = 0; j0 < N; j0 += NC) {
        const int nc = (int)(N - j0 < NC ? N - j0 : NC);
        const int nstrips = (nc + NR - 1) / NR;
        for (long k0 = 0; k0 < K; k0 += KC) {
            const int kc = (int)(K - k0 < KC ? K - k0 : KC);
            pack_b(kc, nc, B + k0 * ldb + j0, ldb, Bp);
#pragma omp parallel
            {
                float *Ap = (float *)aligned_alloc(64, sizeof(float) * (size_t)MC * KC);
                if (!Ap) {
#pragma omp atomic write
                    status = -2;
                }
                long i0;
#pragma omp for schedule(dynamic, 1)
                for (i0 = 0; i0 < M; i0 += MC) {
                    if (!Ap)
                        continue;
                    const int mc = (int)(M - i0 < MC ? M - i0 : MC);
                    pack_a(mc, kc, A + i0 * lda + k0, lda, Ap);
                    for (int si = 0; si < (mc + MR - 1) / MR; ++si) {
                        const int h = mc - si * MR < MR ? mc - si * MR : MR;
                        for (int sj = 0; sj < nstrips; ++sj) {
                            const int w = nc - sj * NR < NR ? nc - sj * NR : NR;
                            micro_kernel(kc, Ap + (long)si * kc * MR, Bp + (long)sj * kc * NR, alpha,
                                         C + (i0 + si * MR) * ldc + j0 + sj * NR, ldc, h, w);
                        }
                    }
                }
                free(Ap);
            }
        }
    }
    free(Bp);
    return status;
}
