/*
 * Plain fp64 CPU reference GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the GPU kernels are checked against.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library: gcc builds
 * it on its own, from this file and attention.c (the attention reference).
 *
 * What it computes (the plain definition, nothing more):
 *     C <- alpha * op(A) * op(B) + beta * C0
 * with every operand decoded exactly to fp64 and every dot product summed in
 * fp64 over k = 0, 1, ..., K-1 in that order, one (i, j) at a time.  Beside the
 * result it returns T(i,j) = sum_k |a(i,k) * b(k,j)|, the scale of the
 * acceptance bound.
 *
 * Sources:
 *  - "B200 GEMM Optimization Ladder", section E step 1 (fix the math
 *    definition, layout, dtype and reference before any level is built) and
 *    steps 2-4 (each level must be element-wise correct against that
 *    reference, including the K tail and the boundary tiles).
 *  - "B200 TMEM Lifecycle Planner", section A1 case 2 (block-scaled MMA: each
 *    operand carries its own scale factors beside the data).  The pages name
 *    no element format; the block size (32 consecutive K elements, one E8M0
 *    scale each) and the element formats (FP8 E4M3 and E5M2, FP6 E2M3 and
 *    E3M2, FP4 E2M1) follow the OCP Microscaling (MX) v1.0 formats.
 *  - The math definition itself is the ordinary BLAS one: C0 is not read when
 *    beta == 0, and A, B are not read when alpha == 0 or K == 0.
 *
 * Number formats (decoded exactly; fp64 holds every value):
 *  - bf16:   the top 16 bits of an IEEE binary32; widen by shifting left 16.
 *  - E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities;
 *            exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN.
 *  - E5M2:   sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent field
 *            31 is infinity (mantissa 0) or NaN; field 0 is subnormal
 *            (m/4 * 2^-14).
 *  - E2M3:   6 bits: sign, 2 exponent bits (bias 1), 3 mantissa bits; no
 *            infinities or NaN; field 0 is subnormal (m/8).
 *  - E3M2:   6 bits: sign, 3 exponent bits (bias 3), 2 mantissa bits; no
 *            infinities or NaN; field 0 is subnormal (m/4 * 2^-2).
 *  - E2M1:   4 bits: sign, 2 exponent bits (bias 1), 1 mantissa bit; no
 *            infinities or NaN; field 0 is subnormal (m/2).
 *  - E8M0:   an unsigned biased exponent, value 2^(b-127); 0xFF is NaN.
 *
 * Storage of the MX element formats: 8-bit formats one byte per element;
 * the 6- and 4-bit formats packed along K, element e of a row at bit offset
 * 6e (4e) of the row's little-endian bit string (so two E2M1 per byte, the
 * lower K in the low nibble, and four E2M3 / E3M2 per three bytes), with
 * leading dimensions in elements.  Packed operands are K-contiguous only
 * (A row-major, B column-major).
 *
 * Leading dimensions are in elements.  a(i,k) lives at A[i*lda + k] when A is
 * row-major and at A[k*lda + i] when it is column-major; b(k,j) lives at
 * B[k*ldb + j] (row-major) or B[j*ldb + k] (column-major); c(i,j) at
 * C[i*ldc + j] or C[j*ldc + i].  MX scales are row-major per operand row or
 * column: SA[i*ld_sa + k/32] and SB[j*ld_sb + k/32].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_E4M3FN = 1, ORACLE_E5M2 = 2, ORACLE_E2M3 = 3, ORACLE_E3M2 = 4,
       ORACLE_E2M1 = 5 };
enum { ORACLE_OUT_F32 = 0, ORACLE_OUT_BF16 = 1 };

double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

double oracle_e4m3fn_to_f64(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* A sign-exponent-mantissa code with no infinities or NaN (the MX 6- and
   4-bit formats): field 0 is subnormal, m / 2^mbits * 2^(1 - bias). */
static double small_float(unsigned code, int ebits, int mbits, int bias)
{
    int sign = (code >> (ebits + mbits)) & 1;
    int e = (code >> mbits) & ((1 << ebits) - 1);
    int m = code & ((1 << mbits) - 1);
    double frac = (double)m / (double)(1 << mbits);
    double mag = e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, e - bias);
    return sign ? -mag : mag;
}

double oracle_e5m2_to_f64(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 2) & 0x1F;
    int m = code & 0x3;
    double mag;
    if (e == 0x1F)
        mag = m == 0 ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m / 4.0, -14);
    else
        mag = ldexp(1.0 + (double)m / 4.0, e - 15);
    return sign ? -mag : mag;
}

double oracle_e2m3_to_f64(uint8_t code) { return small_float(code & 0x3F, 2, 3, 1); }
double oracle_e3m2_to_f64(uint8_t code) { return small_float(code & 0x3F, 3, 2, 3); }
double oracle_e2m1_to_f64(uint8_t code) { return small_float(code & 0xF, 2, 1, 1); }

/* Bits per element of each operand format. */
static int format_bits(int fmt)
{
    switch (fmt) {
    case ORACLE_BF16: return 16;
    case ORACLE_E4M3FN:
    case ORACLE_E5M2: return 8;
    case ORACLE_E2M3:
    case ORACLE_E3M2: return 6;
    case ORACLE_E2M1: return 4;
    default: return 0;
    }
}

/* The code of element idx of an MX operand stored as described above. */
static unsigned mx_code(int fmt, const void *X, int64_t idx)
{
    const uint8_t *b = (const uint8_t *)X;
    int bits = format_bits(fmt);
    if (bits == 8)
        return b[idx];
    int64_t bit = idx * bits;
    unsigned w = b[bit / 8] | ((bit % 8 + bits > 8) ? (unsigned)b[bit / 8 + 1] << 8 : 0u);
    return (w >> (bit % 8)) & ((1u << bits) - 1);
}

static double mx_value(int fmt, unsigned code)
{
    switch (fmt) {
    case ORACLE_E4M3FN: return oracle_e4m3fn_to_f64((uint8_t)code);
    case ORACLE_E5M2: return oracle_e5m2_to_f64((uint8_t)code);
    case ORACLE_E2M3: return oracle_e2m3_to_f64((uint8_t)code);
    case ORACLE_E3M2: return oracle_e3m2_to_f64((uint8_t)code);
    default: return oracle_e2m1_to_f64((uint8_t)code);
    }
}

double oracle_e8m0_to_f64(uint8_t code)
{
    if (code == 0xFF)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

static double f32_bits_to_f64(const void *p, int64_t idx)
{
    float f;
    memcpy(&f, (const char *)p + idx * 4, sizeof f);
    return (double)f;
}

/* a(i,k) of the logical M x K operand, decoded (scale applied for MX). */
static double load_a(int fmt, const void *A, int64_t lda, int col_major,
                     const uint8_t *SA, int64_t ld_sa, int64_t i, int64_t k)
{
    int64_t idx = col_major ? k * lda + i : i * lda + k;
    if (fmt == ORACLE_BF16)
        return oracle_bf16_to_f64(((const uint16_t *)A)[idx]);
    return mx_value(fmt, mx_code(fmt, A, idx)) * oracle_e8m0_to_f64(SA[i * ld_sa + k / 32]);
}

/* b(k,j) of the logical K x N operand, decoded (scale applied for MX). */
static double load_b(int fmt, const void *B, int64_t ldb, int col_major,
                     const uint8_t *SB, int64_t ld_sb, int64_t k, int64_t j)
{
    int64_t idx = col_major ? j * ldb + k : k * ldb + j;
    if (fmt == ORACLE_BF16)
        return oracle_bf16_to_f64(((const uint16_t *)B)[idx]);
    return mx_value(fmt, mx_code(fmt, B, idx)) * oracle_e8m0_to_f64(SB[j * ld_sb + k / 32]);
}

static double load_c0(const void *C0, int64_t ldc, int col_major, int c_dtype,
                      int64_t i, int64_t j)
{
    int64_t idx = col_major ? j * ldc + i : i * ldc + j;
    if (c_dtype == ORACLE_OUT_BF16)
        return oracle_bf16_to_f64(((const uint16_t *)C0)[idx]);
    return f32_bits_to_f64(C0, idx);
}

typedef struct {
    int64_t M, N, K;
    int a_fmt;
    const void *A;
    int64_t lda;
    int a_col_major;
    const uint8_t *SA;
    int64_t ld_sa;
    int b_fmt;
    const void *B;
    int64_t ldb;
    int b_col_major;
    const uint8_t *SB;
    int64_t ld_sb;
    const void *C0;
    int64_t ldc;
    int c_col_major;
    int c_dtype;
    double alpha, beta;
} problem;

/* One output element from already-decoded row a[0..K) and column b[0..K). */
static void entry(const problem *p, const double *a, const double *b,
                  int64_t i, int64_t j, double *out, double *tsum)
{
    double s = 0.0, t = 0.0;
    int use_ab = (p->alpha != 0.0 && p->K > 0);
    if (use_ab) {
        for (int64_t k = 0; k < p->K; ++k) {
            double prod = a[k] * b[k];
            s += prod;
            t += fabs(prod);
        }
    }
    double r = use_ab ? p->alpha * s : 0.0;
    if (p->beta != 0.0)
        r += p->beta * load_c0(p->C0, p->ldc, p->c_col_major, p->c_dtype, i, j);
    *out = r;
    *tsum = t;
}

static int check(const problem *p)
{
    if (p->M < 0 || p->N < 0 || p->K < 0)
        return 1;
    if (format_bits(p->a_fmt) == 0 || format_bits(p->b_fmt) == 0)
        return 1;
    if ((p->a_fmt == ORACLE_BF16) != (p->b_fmt == ORACLE_BF16))
        return 1;
    /* packed formats: K-contiguous rows of whole bytes */
    if (format_bits(p->a_fmt) < 8 && (p->a_col_major || (p->lda * format_bits(p->a_fmt)) % 8))
        return 1;
    if (format_bits(p->b_fmt) < 8 && (!p->b_col_major || (p->ldb * format_bits(p->b_fmt)) % 8))
        return 1;
    if (p->c_dtype != ORACLE_OUT_F32 && p->c_dtype != ORACLE_OUT_BF16)
        return 1;
    int reads_ab = p->alpha != 0.0 && p->K > 0 && p->M > 0 && p->N > 0;
    if (reads_ab && (!p->A || !p->B))
        return 1;
    if (reads_ab && p->a_fmt != ORACLE_BF16 && (!p->SA || !p->SB))
        return 1;
    if (p->beta != 0.0 && p->M > 0 && p->N > 0 && !p->C0)
        return 1;
    return 0;
}

static void decode_row_a(const problem *p, int64_t i, double *a)
{
    if (p->alpha == 0.0)
        return;
    for (int64_t k = 0; k < p->K; ++k)
        a[k] = load_a(p->a_fmt, p->A, p->lda, p->a_col_major, p->SA, p->ld_sa, i, k);
}

static void decode_col_b(const problem *p, int64_t j, double *b)
{
    if (p->alpha == 0.0)
        return;
    for (int64_t k = 0; k < p->K; ++k)
        b[k] = load_b(p->b_fmt, p->B, p->ldb, p->b_col_major, p->SB, p->ld_sb, k, j);
}

/*
 * Rows [row_begin, row_end) of the reference result, every column.
 * Cref and T are (row_end-row_begin) x N, row-major, dense.
 * Returns 0 on success, 1 on bad arguments, 2 when out of memory.
 */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                     int a_fmt, const void *A, int64_t lda, int a_col_major,
                     const uint8_t *SA, int64_t ld_sa,
                     int b_fmt, const void *B, int64_t ldb, int b_col_major,
                     const uint8_t *SB, int64_t ld_sb,
                     const void *C0, int64_t ldc, int c_col_major, int c_dtype,
                     float alpha, float beta,
                     int64_t row_begin, int64_t row_end,
                     double *Cref, double *T)
{
    problem p = {M, N, K, a_fmt, A, lda, a_col_major, SA, ld_sa,
                 b_fmt, B, ldb, b_col_major, SB, ld_sb,
                 C0, ldc, c_col_major, c_dtype, (double)alpha, (double)beta};
    if (check(&p) || row_begin < 0 || row_end > M || row_begin > row_end)
        return 1;
    if (row_begin == row_end || N == 0)
        return 0;
    int64_t kk = K > 0 ? K : 1;
    /* Every column of B decoded once, k-contiguous: Bd[j*K + k] = b(k, j). */
    double *Bd = (double *)malloc((size_t)(N * kk) * sizeof(double));
    if (!Bd)
        return 2;
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        decode_col_b(&p, j, Bd + j * kk);
#pragma omp parallel
    {
        double *a = (double *)malloc((size_t)kk * sizeof(double));
        if (!a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = row_begin; i < row_end; ++i) {
            if (!a)
                continue;
            decode_row_a(&p, i, a);
            int64_t r = i - row_begin;
            for (int64_t j = 0; j < N; ++j)
                entry(&p, a, Bd + j * kk, i, j, Cref + r * N + j, T + r * N + j);
        }
        free(a);
    }
    free(Bd);
    return failed ? 2 : 0;
}

/*
 * Single entries: out[t] = Cref(ii[t], jj[t]) and tsum[t] = T(ii[t], jj[t]).
 * Used to check sampled outputs of full-size problems one by one.
 */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        int a_fmt, const void *A, int64_t lda, int a_col_major,
                        const uint8_t *SA, int64_t ld_sa,
                        int b_fmt, const void *B, int64_t ldb, int b_col_major,
                        const uint8_t *SB, int64_t ld_sb,
                        const void *C0, int64_t ldc, int c_col_major, int c_dtype,
                        float alpha, float beta,
                        int64_t count, const int64_t *ii, const int64_t *jj,
                        double *out, double *tsum)
{
    problem p = {M, N, K, a_fmt, A, lda, a_col_major, SA, ld_sa,
                 b_fmt, B, ldb, b_col_major, SB, ld_sb,
                 C0, ldc, c_col_major, c_dtype, (double)alpha, (double)beta};
    if (check(&p) || count < 0)
        return 1;
    for (int64_t t = 0; t < count; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return 1;
    int64_t kk = K > 0 ? K : 1;
    int failed = 0;
#pragma omp parallel
    {
        double *a = (double *)malloc((size_t)kk * sizeof(double));
        double *b = (double *)malloc((size_t)kk * sizeof(double));
        if (!a || !b) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < count; ++t) {
            if (!a || !b)
                continue;
            decode_row_a(&p, ii[t], a);
            decode_col_b(&p, jj[t], b);
            entry(&p, a, b, ii[t], jj[t], out + t, tsum + t);
        }
        free(a);
        free(b);
    }
    return failed ? 2 : 0;
}

/* Threads the OpenMP runtime will use for the calls above. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
