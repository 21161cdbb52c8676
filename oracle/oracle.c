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
 *   dtype 3  8-bit two's-complement integer (-128 .. 127); every product is
 *            an integer of magnitude at most 2^14, so sums of up to 2^39 of
 *            them are exact in binary64
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

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_I8 = 3 };
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

/* 8-bit two's complement: bit 7 weighs -128, bits 0..6 weigh 1 .. 64. */
double oracle_decode_i8(uint8_t b)
{
    return (double)((int)(b & 0x7f) - (int)(b & 0x80));
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
    if (dtype < ORACLE_F32 || dtype > ORACLE_I8) return ORACLE_BAD_ARG;
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
    if (dtype == ORACLE_I8)
        return oracle_decode_i8(((const uint8_t*)base)[idx]);
    return oracle_decode_bf16(((const uint16_t*)base)[idx]);
}

static int check_args(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                      const void* B, int64_t ldb)
{
    if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
    if (dtype < ORACLE_F32 || dtype > ORACLE_I8) return ORACLE_BAD_ARG;
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

/*
 * Output rounding.  Page "CUDA-Practice 09" (section on why FP32 accumulation
 * is used) has the FP32 accumulator written back as FP32 or rounded as
 * required; the rounding taken here is IEEE round-to-nearest-even: the nearest
 * value of the target format to x, ties to the value whose last significand
 * bit is 0, magnitudes at or beyond the format's overflow threshold to
 * infinity, NaN to a quiet NaN.
 *
 * A finite binary format with p significand bits (hidden bit included) and
 * minimum normal exponent emin represents, in the binade [2^e, 2^(e+1)) for
 * e >= emin, the multiples of q = 2^(e - p + 1); below 2^emin (subnormals) the
 * multiples of 2^(emin - p + 1).  So: take e = max(floor(log2 |x|), emin),
 * q = 2^(e - p + 1), round |x| / q to the nearest integer with ties to even
 * (rint in the default rounding mode), and scale back; a result of 2^p * q has
 * moved into the next binade, which is still exact.  |x| / q is exact: q is a
 * power of two and the quotient stays far below 2^53.
 */
static double round_to_format(double x, int p, int emin, int emax)
{
    if (isnan(x)) return x;
    const double ax = fabs(x);
    /* overflow threshold: the largest finite value plus half its quantum */
    const double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    const double thresh = maxv + ldexp(1.0, emax - p);
    if (ax >= thresh) return x > 0 ? INFINITY : -INFINITY;
    if (ax == 0.0) return x;
    int E;
    frexp(ax, &E); /* ax = m * 2^E, m in [0.5, 1): floor(log2 ax) = E - 1 */
    int e = E - 1;
    if (e < emin) e = emin;
    const double q = ldexp(1.0, e - p + 1);
    const double r = rint(ax / q) * q;
    return x < 0 ? -r : r;
}

/* binary64 -> binary16 bits (p = 11, emin = -14, emax = 15) */
uint16_t oracle_encode_f16(double x)
{
    if (isnan(x)) return 0x7e00;
    const double r = round_to_format(x, 11, -14, 15);
    const uint16_t s = signbit(r) ? 0x8000 : 0;
    const double a = fabs(r);
    if (isinf(a)) return s | 0x7c00;
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -14)) return s | (uint16_t)(a / ldexp(1.0, -24)); /* subnormal: f * 2^-24 */
    int E;
    const double m = frexp(a, &E);                 /* a = m * 2^E, m in [0.5, 1) */
    const int e = E - 1;                           /* a = (1 + f/1024) * 2^e */
    const uint16_t f = (uint16_t)(m * 2048.0 - 1024.0);
    return s | (uint16_t)((e + 15) << 10) | f;
}

/* binary64 -> bfloat16 bits (p = 8, emin = -126, emax = 127) */
uint16_t oracle_encode_bf16(double x)
{
    if (isnan(x)) return 0x7fc0;
    const double r = round_to_format(x, 8, -126, 127);
    const uint16_t s = signbit(r) ? 0x8000 : 0;
    const double a = fabs(r);
    if (isinf(a)) return s | 0x7f80;
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -126)) return s | (uint16_t)(a / ldexp(1.0, -133)); /* f * 2^-133 */
    int E;
    const double m = frexp(a, &E);
    const int e = E - 1;                           /* a = (1 + f/128) * 2^e */
    const uint16_t f = (uint16_t)(m * 256.0 - 128.0);
    return s | (uint16_t)((e + 127) << 7) | f;
}

/* binary64 -> binary32 bits (p = 24, emin = -126, emax = 127) */
uint32_t oracle_encode_f32(double x)
{
    if (isnan(x)) return 0x7fc00000u;
    const double r = round_to_format(x, 24, -126, 127);
    const uint32_t s = signbit(r) ? 0x80000000u : 0;
    const double a = fabs(r);
    if (isinf(a)) return s | 0x7f800000u;
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -126)) return s | (uint32_t)(a / ldexp(1.0, -149));
    int E;
    const double m = frexp(a, &E);
    const int e = E - 1;
    const uint32_t f = (uint32_t)(m * 16777216.0 - 8388608.0);
    return s | ((uint32_t)(e + 127) << 23) | f;
}

/* Encodes n binary64 values into the stored format (4-byte words for dtype 0,
 * 2-byte for 1 and 2). */
int oracle_encode_array(int dtype, int64_t n, const double* in, void* out)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    if (n < 0 || (n > 0 && (!in || !out))) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e) {
        if (dtype == ORACLE_F32)
            ((uint32_t*)out)[e] = oracle_encode_f32(in[e]);
        else if (dtype == ORACLE_F16)
            ((uint16_t*)out)[e] = oracle_encode_f16(in[e]);
        else
            ((uint16_t*)out)[e] = oracle_encode_bf16(in[e]);
    }
    return ORACLE_OK;
}

/*
 * The general output step, element by element (the scaled update of page
 * "matmul_registers.cu", section on the library call, whose alpha and beta
 * multiply the product and the previous C):
 *
 *     out[e]   = alpha * acc[e] + beta * Cold[e]
 *     scale[e] = |alpha| * S[e] + |beta * Cold[e]|
 *
 * acc and S are a product and its scale from oracle_gemm (or _entries); Cold
 * holds n stored elements of dtype c_dtype and is not read when beta == 0
 * (the previous C then takes no part, whatever it holds).  All in binary64;
 * scale may be NULL.
 */
int oracle_epilogue(int64_t n, double alpha, double beta, int c_dtype, const void* Cold,
                    const double* acc, const double* S, double* out, double* scale)
{
    if (c_dtype != ORACLE_F32 && c_dtype != ORACLE_F16 && c_dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    if (n < 0 || (n > 0 && (!acc || !out || (scale && !S) || (beta != 0.0 && !Cold))))
        return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e) {
        const double old = beta != 0.0 ? beta * decode_at(Cold, c_dtype, e) : 0.0;
        out[e] = alpha * acc[e] + old;
        if (scale) scale[e] = fabs(alpha) * S[e] + fabs(old);
    }
    return ORACLE_OK;
}
