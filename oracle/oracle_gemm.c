/*
 * oracle_gemm.c -- the plain CPU oracle for the tiled dense GEMM C = A.B.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never links, loads or calls it; the two share no code.
 *
 * What it computes (the plain definition, no blocking, no reordering):
 *   C[i][j] = sum over k = 0 .. K-1 (increasing) of A[i][k] * B[k][j]
 * with A row-major M x K (leading dimension lda), B row-major K x N
 * (leading dimension ldb), C dense M x N (leading dimension N).
 *   - "Pipeline GPU Kernel", Step 2 (compute/load ratio): one multiply-add
 *     counts as two operations, i.e. the kernel is the plain matrix product.
 *   - "Analyze Kernel Bottleneck", Step 1 (effective GFLOPS of a GEMM is
 *     2*M*N*K over the time): again the plain product of an M x K and a
 *     K x N matrix.
 *   - "Pipeline GPU Kernel", Step 5: the pipelined kernel is checked against a
 *     CPU reference; pipelining only reorders loads, never the arithmetic.
 *
 * Precision:
 *   - INT8 inputs: products and sums in int64 (exact).  The GPU result is
 *     int32; for K <= 131071 no int32 overflow is possible (|a*b| <= 2^14).
 *   - FP16 inputs: each binary16 value is widened exactly to double, every
 *     product of two binary16 values is exact in double, and the sum runs in
 *     double in increasing k.  Alongside it the oracle returns
 *     S[i][j] = sum_k |A[i][k]*B[k][j]|, the scale of the per-element error
 *     bound |C_gpu - C| <= 1e-4 * S.
 *   - FP32 inputs ("Pipeline GPU Kernel", Step 5 lists FP32 scalar FFMA as
 *     the third data type): each binary32 value converts to double exactly,
 *     every product of two binary32 values (48 significant bits at most) is
 *     exact in double, the sum runs in double in increasing k, and S is
 *     returned alongside as for FP16.
 *
 * Parallelism: rows of C are split into contiguous bands, one per thread.
 * Each C[i][j] is still one sequential sum in increasing k, so the thread
 * count never changes a result.
 *
 * Error behaviour: returns 0 on success, -1 on an invalid argument
 * (negative size, leading dimension too small, NULL pointer with a non-empty
 * matrix), -2 if a thread cannot be created.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 encodes zero and subnormals (value f * 2^-24); exponent
 * 31 encodes infinities and NaNs; otherwise the value is
 * (1024 + f) * 2^(e - 25).  Every binary16 value is exact in double. */
double oracle_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* All 65536 binary16 values widened once by oracle_f16_to_f64, so the
 * product loops below look a value up instead of decoding it again. */
static double f16_table[65536];
static pthread_once_t f16_table_once = PTHREAD_ONCE_INIT;

static void f16_table_fill(void)
{
    for (int h = 0; h < 65536; h++)
        f16_table[h] = oracle_f16_to_f64((uint16_t)h);
}

typedef struct {
    int kind; /* 0: int8 -> int64, 1: fp16 -> double (+ S), 2: fp32 -> double (+ S) */
    int64_t row_begin, row_end, N, K;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    void *C;
    double *S;
} band_t;

static void band_i8(const band_t *t)
{
    const int8_t *A = (const int8_t *)t->A;
    const int8_t *B = (const int8_t *)t->B;
    int64_t *C = (int64_t *)t->C;
    for (int64_t i = t->row_begin; i < t->row_end; i++) {
        int64_t *c = C + i * t->N;
        for (int64_t j = 0; j < t->N; j++)
            c[j] = 0;
        /* i-k-j order: for a fixed (i, j) the additions still happen in
         * increasing k, exactly as in the textbook i-j-k loop. */
        for (int64_t k = 0; k < t->K; k++) {
            int64_t a = A[i * t->lda + k];
            const int8_t *b = B + k * t->ldb;
            for (int64_t j = 0; j < t->N; j++)
                c[j] += a * (int64_t)b[j];
        }
    }
}

static void band_f16(const band_t *t)
{
    const uint16_t *A = (const uint16_t *)t->A;
    const uint16_t *B = (const uint16_t *)t->B;
    double *C = (double *)t->C;
    for (int64_t i = t->row_begin; i < t->row_end; i++) {
        double *c = C + i * t->N;
        double *s = t->S ? t->S + i * t->N : NULL;
        for (int64_t j = 0; j < t->N; j++) {
            c[j] = 0.0;
            if (s)
                s[j] = 0.0;
        }
        for (int64_t k = 0; k < t->K; k++) {
            double a = f16_table[A[i * t->lda + k]];
            const uint16_t *b = B + k * t->ldb;
            for (int64_t j = 0; j < t->N; j++) {
                double p = a * f16_table[b[j]];
                c[j] += p;
                if (s)
                    s[j] += fabs(p);
            }
        }
    }
}

/* binary32 inputs: a float converts to double exactly, and the product of
 * two binary32 values (at most 48 significant bits) is exact in double. */
static void band_f32(const band_t *t)
{
    const float *A = (const float *)t->A;
    const float *B = (const float *)t->B;
    double *C = (double *)t->C;
    for (int64_t i = t->row_begin; i < t->row_end; i++) {
        double *c = C + i * t->N;
        double *s = t->S ? t->S + i * t->N : NULL;
        for (int64_t j = 0; j < t->N; j++) {
            c[j] = 0.0;
            if (s)
                s[j] = 0.0;
        }
        for (int64_t k = 0; k < t->K; k++) {
            double a = (double)A[i * t->lda + k];
            const float *b = B + k * t->ldb;
            for (int64_t j = 0; j < t->N; j++) {
                double p = a * (double)b[j];
                c[j] += p;
                if (s)
                    s[j] += fabs(p);
            }
        }
    }
}

static void *band_main(void *arg)
{
    const band_t *t = (const band_t *)arg;
    if (t->kind == 0)
        band_i8(t);
    else if (t->kind == 1)
        band_f16(t);
    else
        band_f32(t);
    return NULL;
}

static int check_args(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                      const void *B, int64_t ldb, const void *C)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1))
        return -1;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (M > 0 && N > 0 && !C))
        return -1;
    return 0;
}

static int run_bands(int kind, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     const void *B, int64_t ldb, void *C, double *S, int nthreads)
{
    if (M == 0 || N == 0)
        return 0;
    pthread_once(&f16_table_once, f16_table_fill);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > M)
        nthreads = (int)M;
    band_t *bands = (band_t *)calloc((size_t)nthreads, sizeof(band_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!bands || !tids) {
        free(bands);
        free(tids);
        return -2;
    }
    int rc = 0, started = 0;
    for (int t = 0; t < nthreads; t++) {
        band_t *b = &bands[t];
        b->kind = kind;
        b->row_begin = M * t / nthreads;
        b->row_end = M * (t + 1) / nthreads;
        b->N = N;
        b->K = K;
        b->A = A;
        b->lda = lda;
        b->B = B;
        b->ldb = ldb;
        b->C = C;
        b->S = S;
    }
    for (int t = 1; t < nthreads; t++) {
        if (pthread_create(&tids[t], NULL, band_main, &bands[t]) != 0) {
            rc = -2;
            break;
        }
        started = t;
    }
    if (rc == 0)
        band_main(&bands[0]);
    for (int t = 1; t <= started; t++)
        pthread_join(tids[t], NULL);
    free(bands);
    free(tids);
    return rc;
}

/* C (M x N, dense int64) = A (M x K int8, lda) . B (K x N int8, ldb). */
int oracle_gemm_i8i64(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                      const int8_t *B, int64_t ldb, int64_t *C, int nthreads)
{
    if (check_args(M, N, K, A, lda, B, ldb, C))
        return -1;
    return run_bands(0, M, N, K, A, lda, B, ldb, C, NULL, nthreads);
}

/* C (M x N, dense double) = A (M x K binary16 bits, lda) . B (K x N, ldb);
 * S (M x N, dense double, may be NULL) = sum_k |A[i][k] * B[k][j]|. */
int oracle_gemm_f16f64(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, double *C, double *S, int nthreads)
{
    if (check_args(M, N, K, A, lda, B, ldb, C))
        return -1;
    return run_bands(1, M, N, K, A, lda, B, ldb, C, S, nthreads);
}

/* C (M x N, dense double) = A (M x K binary32, lda) . B (K x N, ldb);
 * S (M x N, dense double, may be NULL) = sum_k |A[i][k] * B[k][j]|. */
int oracle_gemm_f32f64(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, double *C, double *S, int nthreads)
{
    if (check_args(M, N, K, A, lda, B, ldb, C))
        return -1;
    return run_bands(2, M, N, K, A, lda, B, ldb, C, S, nthreads);
}

/* Single elements of the same product, for matrices too large to multiply
 * whole on the CPU: for each t < count, out[t] = sum_k A[rows[t]][k] *
 * B[k][cols[t]] (increasing k), exactly the value the full routine would put
 * at (rows[t], cols[t]). */
int oracle_gemm_i8i64_at(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                         const int8_t *B, int64_t ldb, const int64_t *rows, const int64_t *cols,
                         int64_t count, int64_t *out)
{
    if (check_args(M, N, K, A, lda, B, ldb, out))
        return -1;
    for (int64_t t = 0; t < count; t++) {
        int64_t i = rows[t], j = cols[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        int64_t acc = 0;
        for (int64_t k = 0; k < K; k++)
            acc += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];
        out[t] = acc;
    }
    return 0;
}

int oracle_gemm_f16f64_at(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb, const int64_t *rows,
                          const int64_t *cols, int64_t count, double *out, double *out_s)
{
    if (check_args(M, N, K, A, lda, B, ldb, out))
        return -1;
    pthread_once(&f16_table_once, f16_table_fill);
    for (int64_t t = 0; t < count; t++) {
        int64_t i = rows[t], j = cols[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double acc = 0.0, sc = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = f16_table[A[i * lda + k]] * f16_table[B[k * ldb + j]];
            acc += p;
            sc += fabs(p);
        }
        out[t] = acc;
        if (out_s)
            out_s[t] = sc;
    }
    return 0;
}

int oracle_gemm_f32f64_at(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          const float *B, int64_t ldb, const int64_t *rows, const int64_t *cols,
                          int64_t count, double *out, double *out_s)
{
    if (check_args(M, N, K, A, lda, B, ldb, out))
        return -1;
    for (int64_t t = 0; t < count; t++) {
        int64_t i = rows[t], j = cols[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double acc = 0.0, sc = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
            acc += p;
            sc += fabs(p);
        }
        out[t] = acc;
        if (out_s)
            out_s[t] = sc;
    }
    return 0;
}
