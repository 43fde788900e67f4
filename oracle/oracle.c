/*
 * CPU oracle for the dense row-major matrix product C = A x B.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * library's own call path never does.  It shares no code, header or table
 * with the GPU library and includes nothing from it.
 *
 * What it computes (the definition, nothing more):
 *   A is M x K, B is K x N, C is M x N, all row-major with packed leading
 *   dimensions (A[i*K+k], B[k*N+j], C[i*N+j]).
 *   C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j].
 *   - "Lesson 8: how a GPU does matrix multiply", section 1 (the element
 *     formula) and section 2 (the row-major index expressions);
 *   - "SGEMM optimisation journey", Level 1 (the same sum, k from 0 to K-1);
 *   - "4. GEMM optimisation", section 4.1 (A is MxK, B is KxN, C is MxN; the
 *     sum starts at zero, so K = 0 yields 0, and C is overwritten).
 *
 * Precision: every product of two binary32 (or two binary16) values is exact
 * in binary64, so each element is the binary64 running sum of exact products,
 * taken in ascending k from +0.0, and rounded once to binary32 with the C
 * cast (round to nearest, ties to even).  Build with -ffp-contract=off so no
 * step is fused.
 *
 * The pages do not fix the accumulator precision (their listings accumulate
 * in float); binary64 accumulation is the reading taken here, so a correct
 * GPU result differs from this one by binary32 accumulation error only, and
 * on small-integer inputs (every partial sum exact) by nothing at all.
 *
 * Parity pins (checked by the CPU test suite, not by re-typing this code):
 * identity and permutation products, rank-1 closed forms, K = 1 against
 * numpy's correctly rounded binary32 product, brute force against exact
 * rational sums on all shapes up to 6x6x6, numpy's binary64 matmul within
 * one binary32 ulp, exact integer products, thread-count determinism, the
 * binary16 decoder against numpy and the bfloat16 decoder against torch over
 * all 65536 bit patterns each.
 *
 * bfloat16 inputs ("Lesson 8: how a GPU does matrix multiply", section 22,
 * lists it among the matrix-unit input formats) are handled exactly like
 * binary16 ones: each value is decoded exactly, every product of two of them
 * is exact in binary64, and the same sum is formed.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_DIM (-1)
#define ORACLE_ERR_ALLOC (-2)
#define ORACLE_ERR_RANGE (-3)

/* IEEE 754 binary16 bit pattern -> exact binary64 value.
 * Layout: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)
 *   exponent 31     : infinity (fraction 0) or NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> exact binary64 value.
 * Layout: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-133
 *   exponent 1..254 : normal,    value = (128 + fraction) * 2^(exponent-134)
 *   exponent 255    : infinity (fraction 0) or NaN. */
double oracle_bf16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 7) & 0xff;
    const int frac = h & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

static int thread_count(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of threads the full-matrix routines use for a given request. */
int oracle_threads(int nthreads) { return thread_count(nthreads); }

/*
 * Full product, binary32 inputs.
 * The loop order is i, then k, then j with one binary64 accumulator per
 * element of the current row.  For every (i, j) the operations are exactly
 * those of the textbook i-j-k loop: start from 0.0, add A[i][k]*B[k][j] for
 * k = 0, 1, ..., K-1, round once.  Rows are independent, so splitting rows
 * across threads cannot change any bit.
 * M = 0 or N = 0 writes nothing; K = 0 writes zeros.
 */
int oracle_gemm_f32(int M, int N, int K, const float *A, const float *B,
                    float *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_DIM;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (!acc)
            failed = 1;
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (!acc)
                continue;
            for (int j = 0; j < N; ++j)
                acc[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const double a = (double)A[(size_t)i * K + k];
                const float *brow = B + (size_t)k * N;
                for (int j = 0; j < N; ++j)
                    acc[j] += a * (double)brow[j];
            }
            for (int j = 0; j < N; ++j)
                C[(size_t)i * N + j] = (float)acc[j];
        }
        free(acc);
    }
    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;
}

/*
 * Full product, binary16 inputs given as raw bit patterns, binary32 output.
 * Each input is decoded exactly to binary64 by oracle_f16_to_f64 (through a
 * 65536-entry table of its results), then the same sum as above is formed.
 */
int oracle_gemm_f16(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                    float *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_DIM;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    double *dec = (double *)malloc(65536 * sizeof(double));
    if (!dec)
        return ORACLE_ERR_ALLOC;
    for (int h = 0; h < 65536; ++h)
        dec[h] = oracle_f16_to_f64((uint16_t)h);
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (!acc)
            failed = 1;
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (!acc)
                continue;
            for (int j = 0; j < N; ++j)
                acc[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const double a = dec[A[(size_t)i * K + k]];
                const uint16_t *brow = B + (size_t)k * N;
                for (int j = 0; j < N; ++j)
                    acc[j] += a * dec[brow[j]];
            }
            for (int j = 0; j < N; ++j)
                C[(size_t)i * N + j] = (float)acc[j];
        }
        free(acc);
    }
    free(dec);
    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;
}

/*
 * Full product, bfloat16 inputs given as raw bit patterns, binary32 output:
 * the binary16 routine with oracle_bf16_to_f64 as the decoder.
 */
int oracle_gemm_bf16(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                     float *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_DIM;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    double *bdec = (double *)malloc(65536 * sizeof(double));
    if (!bdec)
        return ORACLE_ERR_ALLOC;
    for (int h = 0; h < 65536; ++h)
        bdec[h] = oracle_bf16_to_f64((uint16_t)h);
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (!acc)
            failed = 1;
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (!acc)
                continue;
            for (int j = 0; j < N; ++j)
                acc[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const double a = bdec[A[(size_t)i * K + k]];
                const uint16_t *brow = B + (size_t)k * N;
                for (int j = 0; j < N; ++j)
                    acc[j] += a * bdec[brow[j]];
            }
            for (int j = 0; j < N; ++j)
                C[(size_t)i * N + j] = (float)acc[j];
        }
        free(acc);
    }
    free(bdec);
    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;
}

/*
 * Selected elements only: out[t] = C[rows[t]][cols[t]], each formed as the
 * plain dot product of row rows[t] of A with column cols[t] of B in ascending
 * k.  Same operation sequence as the full routines, so the same bits; used
 * where the full product would take too long on the host.
 */
int oracle_gemm_f32_at(int M, int N, int K, const float *A, const float *B,
                       int64_t count, const int64_t *rows, const int64_t *cols,
                       float *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_ERR_DIM;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_ERR_DIM;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += (double)A[(size_t)i * K + k] * (double)B[(size_t)k * N + j];
        out[t] = (float)acc;
    }
    return ORACLE_OK;
}

int oracle_gemm_f16_at(int M, int N, int K, const uint16_t *A,
                       const uint16_t *B, int64_t count, const int64_t *rows,
                       const int64_t *cols, float *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_ERR_DIM;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_ERR_DIM;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += oracle_f16_to_f64(A[(size_t)i * K + k]) *
                   oracle_f16_to_f64(B[(size_t)k * N + j]);
        out[t] = (float)acc;
    }
    return ORACLE_OK;
}

int oracle_gemm_bf16_at(int M, int N, int K, const uint16_t *A,
                        const uint16_t *B, int64_t count, const int64_t *rows,
                        const int64_t *cols, float *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_ERR_DIM;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_ERR_DIM;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += oracle_bf16_to_f64(A[(size_t)i * K + k]) *
                   oracle_bf16_to_f64(B[(size_t)k * N + j]);
        out[t] = (float)acc;
    }
    return ORACLE_OK;
}

/*
 * General layouts and scaling: C = alpha * op(A) * op(B) + beta * C, the form
 * "Lesson 8: how a GPU does matrix multiply", section 28, says libraries
 * expose (its section 21 writes the matrix unit's D = A x B + C).
 *   op(A)[i][k] = A[i*lda + k]      (opA == 0)  or  A[k*lda + i]  (opA == 1)
 *   op(B)[k][j] = B[k*ldb + j]      (opB == 0)  or  B[j*ldb + k]  (opB == 1)
 *   C[i][j]     = C[i*ldc + j]
 * Each element: the binary64 sum of the exact products in ascending k from
 * +0.0, then alpha * sum + beta * C_in in binary64 (C_in is not read when
 * beta == 0), rounded once to binary32.  `in` selects the input format:
 * 0 binary32, 1 binary16 bits, 2 bfloat16 bits.
 */
static double oracle_in_value(int in, const void *p, size_t idx)
{
    if (in == 0)
        return (double)((const float *)p)[idx];
    const uint16_t h = ((const uint16_t *)p)[idx];
    return in == 1 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);
}

int oracle_gemm_ex(int in, int opA, int opB, int M, int N, int K, double alpha,
                   const void *A, int lda, const void *B, int ldb, double beta,
                   float *C, int ldc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || in < 0 || in > 2 || opA < 0 || opA > 1 || opB < 0 || opB > 1)
        return ORACLE_ERR_DIM;
    if (lda < (opA ? M : K) || ldb < (opB ? K : N) || ldc < N)
        return ORACLE_ERR_DIM;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static)
    for (int i = 0; i < M; ++i) {
        for (int j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                const size_t ia = opA ? (size_t)k * lda + i : (size_t)i * lda + k;
                const size_t ib = opB ? (size_t)j * ldb + k : (size_t)k * ldb + j;
                acc += oracle_in_value(in, A, ia) * oracle_in_value(in, B, ib);
            }
            double v = alpha * acc;
            if (beta != 0.0)
                v += beta * (double)C[(size_t)i * ldc + j];
            C[(size_t)i * ldc + j] = (float)v;
        }
    }
    return ORACLE_OK;
}

/*
 * 8-bit inputs ("Lesson 8: how a GPU does matrix multiply", section 22 lists
 * FP8 and INT8 among the matrix units' input formats).
 *
 * OCP FP8 E4M3 (the "FN" variant, no infinities): 1 sign bit, 4 exponent
 * bits (bias 7), 3 fraction bits.
 *   exponent 0             : subnormal, value = fraction * 2^-9
 *   exponent 1..15         : normal,    value = (8 + fraction) * 2^(exponent-10)
 *   exponent 15, fraction 7: NaN (the format's only non-finite code).
 */
double oracle_e4m3_to_f64(uint8_t b)
{
    const int sign = (b >> 7) & 1;
    const int expo = (b >> 3) & 0xf;
    const int frac = b & 0x7;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -9);
    else if (expo == 15 && frac == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + frac), expo - 10);
    return sign ? -v : v;
}

/*
 * OCP FP8 E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits.
 *   exponent 0     : subnormal, value = fraction * 2^-16
 *   exponent 1..30 : normal,    value = (4 + fraction) * 2^(exponent-17)
 *   exponent 31    : infinity (fraction 0) or NaN.
 */
double oracle_e5m2_to_f64(uint8_t b)
{
    const int sign = (b >> 7) & 1;
    const int expo = (b >> 2) & 0x1f;
    const int frac = b & 0x3;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -16);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + frac), expo - 17);
    return sign ? -v : v;
}

/*
 * Full product of two 8-bit floating-point matrices given as codes, binary32
 * output: the binary64 sum in ascending k of the exact products of the
 * decoded values, rounded once.  `fmt` 0 is E4M3, 1 is E5M2.
 */
static int gemm_fp8(int fmt, int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C,
                    int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_DIM;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    double dec[256];
    for (int b = 0; b < 256; ++b)
        dec[b] = fmt == 0 ? oracle_e4m3_to_f64((uint8_t)b) : oracle_e5m2_to_f64((uint8_t)b);
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (!acc)
            failed = 1;
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (!acc)
                continue;
            for (int j = 0; j < N; ++j)
                acc[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const double a = dec[A[(size_t)i * K + k]];
                const uint8_t *brow = B + (size_t)k * N;
                for (int j = 0; j < N; ++j)
                    acc[j] += a * dec[brow[j]];
            }
            for (int j = 0; j < N; ++j)
                C[(size_t)i * N + j] = (float)acc[j];
        }
        free(acc);
    }
    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;
}

int oracle_gemm_e4m3(int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C, int nthreads)
{
    return gemm_fp8(0, M, N, K, A, B, C, nthreads);
}

int oracle_gemm_e5m2(int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C, int nthreads)
{
    return gemm_fp8(1, M, N, K, A, B, C, nthreads);
}

/*
 * INT8 inputs, exact integer result: C[i][j] = sum_k A[i][k] B[k][j] as a
 * 64-bit integer, stored as int32.  A result outside the int32 range is an
 * error (ORACLE_ERR_RANGE): it cannot occur for K <= 131072.
 */
int oracle_gemm_i8(int M, int N, int K, const int8_t *A, const int8_t *B, int32_t *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_DIM;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        int64_t *acc = (int64_t *)malloc((size_t)N * sizeof(int64_t));
        if (!acc)
            failed |= 1;
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (!acc)
                continue;
            for (int j = 0; j < N; ++j)
                acc[j] = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t a = A[(size_t)i * K + k];
                const int8_t *brow = B + (size_t)k * N;
                for (int j = 0; j < N; ++j)
                    acc[j] += a * brow[j];
            }
            for (int j = 0; j < N; ++j) {
                if (acc[j] > INT32_MAX || acc[j] < INT32_MIN)
                    failed |= 2;
                C[(size_t)i * N + j] = (int32_t)acc[j];
            }
        }
        free(acc);
    }
    return (failed & 1) ? ORACLE_ERR_ALLOC : (failed & 2) ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* Selected elements of the 8-bit products, one dot product each (same
 * operation sequence as the full routines, so the same bits). */
int oracle_gemm_fp8_at(int fmt, int M, int N, int K, const uint8_t *A, const uint8_t *B,
                       int64_t count, const int64_t *rows, const int64_t *cols, float *out,
                       int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0 || fmt < 0 || fmt > 1)
        return ORACLE_ERR_DIM;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_ERR_DIM;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            const uint8_t a = A[(size_t)i * K + k], b = B[(size_t)k * N + j];
            acc += fmt == 0 ? oracle_e4m3_to_f64(a) * oracle_e4m3_to_f64(b)
                            : oracle_e5m2_to_f64(a) * oracle_e5m2_to_f64(b);
        }
        out[t] = (float)acc;
    }
    return ORACLE_OK;
}

int oracle_gemm_i8_at(int M, int N, int K, const int8_t *A, const int8_t *B, int64_t count,
                      const int64_t *rows, const int64_t *cols, int32_t *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_ERR_DIM;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_ERR_DIM;
    int failed = 0;
#pragma omp parallel for num_threads(thread_count(nthreads)) schedule(static) reduction(| : failed)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        int64_t acc = 0;
        for (int k = 0; k < K; ++k)
            acc += (int64_t)A[(size_t)i * K + k] * B[(size_t)k * N + j];
        if (acc > INT32_MAX || acc < INT32_MIN)
            failed = 1;
        out[t] = (int32_t)acc;
    }
    return failed ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/*
 * Two-dimensional convolution as deep-learning frameworks define it (a
 * cross-correlation), the operator "Lesson 8: how a GPU does matrix
 * multiply" names as the next lesson (convolution as matrix multiplication;
 * input and output feature maps and weights; channel, height, width; direct
 * convolution against im2col).  Written out directly, with no im2col:
 *   x: N x C x H x W, w: K x C x R x S, y: N x K x P x Q (row-major, NCHW),
 *   P = (H + 2 ph - dh (R - 1) - 1) / sh + 1, Q likewise with W, S, pw, sw, dw,
 *   y[n][k][p][q] = sum over c, r, s (in that order, ascending) of
 *       x[n][c][p sh - ph + r dh][q sw - pw + s dw] * w[k][c][r][s],
 *   terms whose input row or column falls outside the image being zero.
 * Each element is the binary64 sum of the exact products, rounded once to
 * binary32.  `in` selects the input format: 0 binary32, 1 binary16 bits,
 * 2 bfloat16 bits.
 */
int oracle_conv2d(int in, int N, int C, int H, int W, int K, int R, int S, int sh, int sw, int ph, int pw,
                  int dh, int dw, const void *x, const void *w, float *y, int nthreads)
{
    if (N < 0 || C < 0 || H < 0 || W < 0 || K < 0 || R < 1 || S < 1 || sh < 1 || sw < 1 || ph < 0 ||
        pw < 0 || dh < 1 || dw < 1 || in < 0 || in > 2)
        return ORACLE_ERR_DIM;
    const int P = (H + 2 * ph - dh * (R - 1) - 1) / sh + 1;
    const int Q = (W + 2 * pw - dw * (S - 1) - 1) / sw + 1;
    if (H + 2 * ph - dh * (R - 1) - 1 < 0 || W + 2 * pw - dw * (S - 1) - 1 < 0)
        return ORACLE_ERR_DIM;
#pragma omp parallel for collapse(2) num_threads(thread_count(nthreads)) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (int p = 0; p < P; ++p)
                for (int q = 0; q < Q; ++q) {
                    double acc = 0.0;
                    for (int c = 0; c < C; ++c)
                        for (int r = 0; r < R; ++r)
                            for (int s = 0; s < S; ++s) {
                                const int h = p * sh - ph + r * dh, v = q * sw - pw + s * dw;
                                if (h < 0 || h >= H || v < 0 || v >= W)
                                    continue;
                                const size_t ix = (((size_t)n * C + c) * H + h) * W + v;
                                const size_t iw = (((size_t)k * C + c) * R + r) * S + s;
                                acc += oracle_in_value(in, x, ix) * oracle_in_value(in, w, iw);
                            }
                    y[(((size_t)n * K + k) * P + p) * Q + q] = (float)acc;
                }
    return ORACLE_OK;
}
