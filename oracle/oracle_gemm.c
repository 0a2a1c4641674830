/*
 * oracle_gemm.c -- plain CPU reference for dense C = alpha*A*B + beta*C, accumulated in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product (the HIP library under
 * register_tiled_matrix_amd/) never calls it, and the two share no source, header or helper.
 *
 * What is computed (the definition, written out):
 *
 *     C_ref[i][j] = alpha * sum_{k=0..K-1} A[i][k] * B[k][j]  +  beta * C_in[i][j]
 *
 *   - "Understanding Register Tiling" (blog.csdn.net/sweet_ran, "【infra之路】理解 Register
 *     Tiling"), opening section on what one thread does in the shared-memory version: an
 *     output element C[row][col] is the running sum over k of A[row][k]*B[k][col]. The
 *     section on the key loop shows the register-tiled version forming exactly the same
 *     products (threadResults[m][n] accumulates regA[m]*regB[n]); only where the operands
 *     are read from changes, so the result is the textbook product up to rounding order.
 *   - alpha and beta: the pages compute C = A*B only. The alpha/beta form follows the BLAS
 *     convention: beta == 0 means C_in is not read (NaN in it cannot leak through);
 *     alpha == 0 or K == 0 means A and B are not read and C = beta*C_in.
 *
 * Arithmetic: every input value is widened exactly to double (fp32 directly, bf16 by
 * placing its 16 bits on top of an fp32 word, fp16 by decoding IEEE 754 binary16: sign,
 * 5-bit exponent with bias 15, 10-bit fraction, subnormals at 2^-24 steps); products and
 * the k-sum are formed in double,
 * k in natural order 0,1,...,K-1 for every element. This file is compiled with
 * -ffp-contract=off so each step is one IEEE double multiply or add.
 *
 * Alongside the result the oracle returns, per element, the magnitude that scales the
 * parity bound:
 *
 *     mag[i][j] = |alpha| * sum_k |A[i][k]*B[k][j]|  +  |beta * C_in[i][j]|
 *
 * Layouts: A is M x K row-major with leading dimension lda >= K. For the fp32 entry points
 * B is K x N row-major (ldb >= N); for the bf16 and fp16 entry points B is K x N column-major
 * (element (k, n) at B[n*ldb + k], ldb >= K). C_in is M x N row-major (ldc >= N) and may be
 * NULL when beta == 0. Outputs are dense M x N row-major doubles (or n values for the
 * sampled-entry variants). Return value: 0, or -1 on an invalid size.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31, (-1)^s * 2^-14 * f/1024
 * for e == 0, infinities and NaNs for e == 31. Every value is a small integer times a power
 * of two, so the result is exact in double. */
static double widen_f16(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* widen_f16 of every 16-bit pattern, filled before a product's loops (the same values as
 * calling widen_f16 per element, without decoding each operand K times). */
static double f16_value[65536];

static void fill_f16_values(void)
{
    for (long h = 0; h < 65536; ++h)
        f16_value[h] = widen_f16((uint16_t)h);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int bad_sizes(long M, long N, long K)
{
    return M < 0 || N < 0 || K < 0;
}

/* Full product, fp32 operands, row-major B. */
int oracle_gemm_f32(long M, long N, long K, double alpha,
                    const float *A, long lda, const float *B, long ldb,
                    double beta, const float *C, long ldc,
                    double *out, double *mag)
{
    if (bad_sizes(M, N, K))
        return -1;
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *o = out + i * N;
        double *g = mag ? mag + i * N : 0;
        for (long j = 0; j < N; ++j) {
            o[j] = 0.0;
            if (g)
                g[j] = 0.0;
        }
        if (alpha != 0.0) {
            /* i-k-j order: each o[j] still receives its terms for k = 0, 1, 2, ... in turn. */
            for (long k = 0; k < K; ++k) {
                double a = (double)A[i * lda + k];
                const float *brow = B + k * ldb;
                for (long j = 0; j < N; ++j) {
                    double p = a * (double)brow[j];
                    o[j] += p;
                    if (g)
                        g[j] += fabs(p);
                }
            }
        }
        for (long j = 0; j < N; ++j) {
            double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
            o[j] = alpha * o[j] + bc;
            if (g)
                g[j] = fabs(alpha) * g[j] + fabs(bc);
        }
    }
    return 0;
}

/* Full product, bf16 operands (uint16 bit patterns), column-major B, fp32 C_in. */
int oracle_gemm_bf16(long M, long N, long K, double alpha,
                     const uint16_t *A, long lda, const uint16_t *B, long ldb,
                     double beta, const float *C, long ldc,
                     double *out, double *mag)
{
    if (bad_sizes(M, N, K))
        return -1;
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        for (long j = 0; j < N; ++j) {
            double s = 0.0, t = 0.0;
            if (alpha != 0.0) {
                const uint16_t *arow = A + i * lda;
                const uint16_t *bcol = B + j * ldb;
                for (long k = 0; k < K; ++k) {
                    double p = widen_bf16(arow[k]) * widen_bf16(bcol[k]);
                    s += p;
                    t += fabs(p);
                }
            }
            double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
            out[i * N + j] = alpha * s + bc;
            if (mag)
                mag[i * N + j] = fabs(alpha) * t + fabs(bc);
        }
    }
    return 0;
}

/* Sampled entries (I[e], J[e]) of the fp32 product; same arithmetic as oracle_gemm_f32. */
int oracle_gemm_f32_entries(long M, long N, long K, double alpha,
                            const float *A, long lda, const float *B, long ldb,
                            double beta, const float *C, long ldc,
                            long n, const long *I, const long *J,
                            double *out, double *mag)
{
    if (bad_sizes(M, N, K) || n < 0)
        return -1;
    for (long e = 0; e < n; ++e)
        if (I[e] < 0 || I[e] >= M || J[e] < 0 || J[e] >= N)
            return -1;
    long e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n; ++e) {
        long i = I[e], j = J[e];
        double s = 0.0, t = 0.0;
        if (alpha != 0.0) {
            for (long k = 0; k < K; ++k) {
                double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
                s += p;
                t += fabs(p);
            }
        }
        double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
        out[e] = alpha * s + bc;
        if (mag)
            mag[e] = fabs(alpha) * t + fabs(bc);
    }
    return 0;
}

/* Sampled entries of the bf16 product (column-major B). */
int oracle_gemm_bf16_entries(long M, long N, long K, double alpha,
                             const uint16_t *A, long lda, const uint16_t *B, long ldb,
                             double beta, const float *C, long ldc,
                             long n, const long *I, const long *J,
                             double *out, double *mag)
{
    if (bad_sizes(M, N, K) || n < 0)
        return -1;
    for (long e = 0; e < n; ++e)
        if (I[e] < 0 || I[e] >= M || J[e] < 0 || J[e] >= N)
            return -1;
    long e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n; ++e) {
        long i = I[e], j = J[e];
        double s = 0.0, t = 0.0;
        if (alpha != 0.0) {
            const uint16_t *arow = A + i * lda;
            const uint16_t *bcol = B + j * ldb;
            for (long k = 0; k < K; ++k) {
                double p = widen_bf16(arow[k]) * widen_bf16(bcol[k]);
                s += p;
                t += fabs(p);
            }
        }
        double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
        out[e] = alpha * s + bc;
        if (mag)
            mag[e] = fabs(alpha) * t + fabs(bc);
    }
    return 0;
}

/* Full product, fp16 operands (uint16 bit patterns), column-major B, fp32 C_in. */
int oracle_gemm_f16(long M, long N, long K, double alpha,
                    const uint16_t *A, long lda, const uint16_t *B, long ldb,
                    double beta, const float *C, long ldc,
                    double *out, double *mag)
{
    if (bad_sizes(M, N, K))
        return -1;
    fill_f16_values();
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        for (long j = 0; j < N; ++j) {
            double s = 0.0, t = 0.0;
            if (alpha != 0.0) {
                const uint16_t *arow = A + i * lda;
                const uint16_t *bcol = B + j * ldb;
                for (long k = 0; k < K; ++k) {
                    double p = f16_value[arow[k]] * f16_value[bcol[k]];
                    s += p;
                    t += fabs(p);
                }
            }
            double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
            out[i * N + j] = alpha * s + bc;
            if (mag)
                mag[i * N + j] = fabs(alpha) * t + fabs(bc);
        }
    }
    return 0;
}

/* Sampled entries of the fp16 product (column-major B). */
int oracle_gemm_f16_entries(long M, long N, long K, double alpha,
                            const uint16_t *A, long lda, const uint16_t *B, long ldb,
                            double beta, const float *C, long ldc,
                            long n, const long *I, const long *J,
                            double *out, double *mag)
{
    if (bad_sizes(M, N, K) || n < 0)
        return -1;
    for (long e = 0; e < n; ++e)
        if (I[e] < 0 || I[e] >= M || J[e] < 0 || J[e] >= N)
            return -1;
    fill_f16_values();
    long e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n; ++e) {
        long i = I[e], j = J[e];
        double s = 0.0, t = 0.0;
        if (alpha != 0.0) {
            const uint16_t *arow = A + i * lda;
            const uint16_t *bcol = B + j * ldb;
            for (long k = 0; k < K; ++k) {
                double p = f16_value[arow[k]] * f16_value[bcol[k]];
                s += p;
                t += fabs(p);
            }
        }
        double bc = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
        out[e] = alpha * s + bc;
        if (mag)
            mag[e] = fabs(alpha) * t + fabs(bc);
    }
    return 0;
}
