/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain CPU definition of the dense matrix product that the GPU library
 * computes, accumulated in IEEE binary64.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the GPU
 * product path never calls it and shares no source with it.
 *
 * What it computes (page "Tensor cores and matrix operations", section
 * "Traditional Approach: Element-by-Element"): for A of M x K and B of K x N,
 *
 *     C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 *
 * over the same rounded input values the GPU reads (page "04-wmma-matmul.cu",
 * the CPU reference built from the half values cast back).  Every element
 * is decoded to an exact binary64 value; the product of two decoded inputs
 * is exact in binary64 (at most 24 + 24 significant bits), and the K products
 * are added in ascending k into one binary64 accumulator.  The loop order is
 * row, k, column, the order of the fp64 CPU reference on page
 * "matmul_registers.cu": each element still receives its terms in ascending
 * k, so the result equals the row, column, k order exactly.
 *
 * Alongside C the oracle returns S[i][j] = sum_k |A[i][k] * B[k][j]|, the
 * scale of the forward error bound of a dot product, which the tests use as
 * the tolerance scale.
 *
 * Input encodings (decoded here from their bit layouts, not from any vendor
 * header):
 *   dtype 0  IEEE binary32: sign, 8-bit exponent (bias 127), 23-bit fraction
 *   dtype 1  IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction
 *   dtype 2  bfloat16: the upper 16 bits of a binary32 word
 * All arrays are row-major with leading dimensions lda, ldb (in elements).
 * C and S are written densely with leading dimension N.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -lm
 * (-ffp-contract=off keeps each multiply and add a separately rounded binary64
 * operation; the products are exact either way.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEMORY = 2 };

/* binary16: value = (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31,
 * (-1)^s * 2^-14 * (f/1024) for e == 0, infinity or NaN for e == 31. */
double oracle_decode_f16(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);            /* f/1024 * 2^-14 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1024+f)/1024 * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: value = (-1)^s * 2^(e-127) * (1 + f/128) for 0 < e < 255,
 * (-1)^s * 2^-126 * (f/128) for e == 0, infinity or NaN for e == 255. */
double oracle_decode_bf16(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int e = (h >> 7) & 0xff;
    const int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);           /* f/128 * 2^-126 */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134); /* (128+f)/128 * 2^(e-127) */
    return s ? -v : v;
}

/* binary32 widened to binary64: exact. */
double oracle_decode_f32(uint32_t w)
{
    float x;
    memcpy(&x, &w, sizeof x);
    return (double)x;
}

static double decode_at(const void* base, int dtype, int64_t idx);

/* Decodes n stored elements of the given dtype to binary64. */
int oracle_decode_array(int dtype, int64_t n, const void* in, double* out)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    if (n < 0 || (n > 0 && (!in || !out))) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e) out[e] = decode_at(in, dtype, e);
    return ORACLE_OK;
}

static double decode_at(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return oracle_decode_f32(((const uint32_t*)base)[idx]);
    if (dtype == ORACLE_F16)
        return oracle_decode_f16(((const uint16_t*)base)[idx]);
    return oracle_decode_bf16(((const uint16_t*)base)[idx]);
}

static int check_args(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                      const void* B, int64_t ldb)
{
    if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (M > 0 && K > 0 && !A) return ORACLE_BAD_ARG;
    if (K > 0 && N > 0 && !B) return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Threads the last parallel region may use (1 without OpenMP). */
int oracle_max_threads(int nthreads)
{
#ifdef _OPENMP
    set_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Full product: C (M x N, dense) and S (M x N, dense, may be NULL).
 * B is decoded once into binary64; each row of C is independent, so rows
 * are shared among threads, and no sum is split or reordered.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                const void* B, int64_t ldb, double* C, double* S, int nthreads)
{
    int st = check_args(M, N, K, dtype, A, lda, B, ldb);
    if (st != ORACLE_OK) return st;
    if (M > 0 && N > 0 && !C) return ORACLE_BAD_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;

    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return ORACLE_NO_MEMORY;
    }
    set_threads(nthreads);

#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = decode_at(B, dtype, k * ldb + j);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        double* s = S ? S + i * N : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (s)
            for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = decode_at(A, dtype, i * lda + k);
            const double* b = Bd + k * N;
            if (s) {
                for (int64_t j = 0; j < N; ++j) {
                    const double p = a * b[j];
                    c[j] += p;
                    s[j] += fabs(p);
                }
            } else {
                for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
            }
        }
    }
    free(Bd);
    return ORACLE_OK;
}

/*
 * Selected entries, one dot product each: for e in [0, n),
 *   C[e] = sum_k A[rows[e]][k] * B[k][cols[e]],  S[e] = sum_k |...|,
 * the same ascending-k binary64 sum as oracle_gemm.  Used where the full
 * product is too large to form on the CPU.
 */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                        const void* B, int64_t ldb, int64_t n, const int64_t* rows,
                        const int64_t* cols, double* C, double* S, int nthreads)
{
    int st = check_args(M, N, K, dtype, A, lda, B, ldb);
    if (st != ORACLE_OK) return st;
    if (n < 0 || (n > 0 && (!rows || !cols || !C))) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return ORACLE_BAD_ARG;
    set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = 0; e < n; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = decode_at(A, dtype, i * lda + k) * decode_at(B, dtype, k * ldb + j);
            c += p;
            s += fabs(p);
        }
        C[e] = c;
        if (S) S[e] = s;
    }
    return ORACLE_OK;
}
