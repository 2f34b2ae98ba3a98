/*
 * oracle_gemm.c -- CPU reference for dense GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with the
 * GPU library; the two are built and linked separately.
 *
 * What it computes is the plain definition of the product, written out:
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *
 * (page "4.1 Tối ưu hiệu năng toán tử GEMM trên CUDA", §1.1 and the naive
 * kernel of §3.1; MUSA learning center lesson m11-l5, case 4 "GEMM 优化",
 * problem statement; page "Operator & Runtime", §5.2.1 loop nest).  All three
 * matrices are row-major; lda/ldb/ldc are row strides in elements.
 *
 * Precision: every input element is widened exactly to double, the products
 * of two float (or bf16) values are exact in double (24+24 significant bits
 * < 53), and the sum runs in double with k ascending for every (i,j).  The
 * result is returned unrounded, in double.  The loop order is i, then k, then
 * j over a double row accumulator -- the same per-element summation order as
 * the i-j-k nest of the pages, arranged so the inner loop walks contiguous
 * rows of B ("Operator & Runtime", §5.2.1, discussion of loop order).
 *
 * Rows of C are independent; OpenMP splits the i loop, so every element is
 * produced by one thread in the same order regardless of thread count.
 *
 * bf16 handling: a bf16 value is the upper 16 bits of an IEEE binary32
 * pattern, so widening places the 16 bits in the high half of a float.
 * The rounding helper turns a binary32 value into bf16 by round to nearest,
 * ties to even, as the pages require a single round_to_bf16 of the finished
 * FP32 accumulator ("Operator & Runtime", §5.2.2 and §5.4.3); it is
 * written from the bit-level definition of that rounding.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

static double widen_bf16(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* C (double, ldc) := A (float, lda) * B (float, ldb). */
void oracle_gemm_f64_from_f32(int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda,
                              const float *B, int64_t ldb,
                              double *C, int64_t ldc)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *acc = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
        }
    }
}

/* C (double, ldc) := A (bf16 bits, lda) * B (bf16 bits, ldb). */
void oracle_gemm_f64_from_bf16(int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               double *C, int64_t ldc)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *acc = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = widen_bf16(A[i * lda + k]);
            const uint16_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) acc[j] += a * widen_bf16(brow[j]);
        }
    }
}

/* Batched form: entry b uses A + b*sA, B + b*sB, C + b*sC (elements);
 * each entry is the single product above ("4.1 Tối ưu hiệu năng toán tử GEMM
 * trên CUDA", §1.2 names batched GEMM for multi-head attention). */
void oracle_gemm_f64_batched_from_bf16(int64_t batch, int64_t M, int64_t N, int64_t K,
                                       const uint16_t *A, int64_t lda, int64_t sA,
                                       const uint16_t *B, int64_t ldb, int64_t sB,
                                       double *C, int64_t ldc, int64_t sC)
{
    for (int64_t b = 0; b < batch; ++b)
        oracle_gemm_f64_from_bf16(M, N, K, A + b * sA, lda, B + b * sB, ldb,
                                  C + b * sC, ldc);
}

/* One output element, for spot checks at full size: sum_k A[i][k]*B[k][j]
 * with k ascending, in double. */
double oracle_dot_f64_from_bf16(int64_t K, const uint16_t *arow, const uint16_t *B,
                                int64_t ldb, int64_t j)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += widen_bf16(arow[k]) * widen_bf16(B[k * ldb + j]);
    return acc;
}

double oracle_dot_f64_from_f32(int64_t K, const float *arow, const float *B,
                               int64_t ldb, int64_t j)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += (double)arow[k] * (double)B[k * ldb + j];
    return acc;
}

/* binary32 -> bf16 bits, round to nearest, ties to even.
 * Finite values: keep the upper 16 bits, add one unit in the last kept place
 * when the dropped 16 bits exceed half a unit, or equal half a unit and the
 * kept part is odd.  A carry out of the significand moves into the exponent,
 * which is how the largest finite values round up to infinity.  Infinities
 * keep their sign; a NaN stays a NaN (its quiet bit is set so that dropping
 * low payload bits cannot turn it into an infinity). */
uint16_t oracle_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const uint32_t exp_bits = (u >> 23) & 0xffu;
    const uint32_t man_bits = u & 0x7fffffu;
    if (exp_bits == 0xffu) {
        if (man_bits != 0) return (uint16_t)((u >> 16) | 0x0040u); /* NaN */
        return (uint16_t)(u >> 16);                                /* +-Inf */
    }
    uint32_t kept = u >> 16;
    const uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

void oracle_round_bf16_array(int64_t n, const float *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

/* ---------------------------------------------------------------------
 * Fused epilogues of page "Operator & Runtime": the activation of §5.4.2
 * (Y = SiLU(A.W)) and the SwiGLU product of §5.3.1 (Z = SiLU(G) (.) U with
 * G = X.W_g, U = X.W_u).  §5.4.3 requires the rounding of the unfused
 * program to survive fusion: the FP32 product is rounded to bf16 before the
 * activation.  For SwiGLU the unfused program keeps G, U and T = SiLU(G) as
 * bf16 tensors, so each of them is rounded to bf16 once; the final output is
 * returned unrounded (double), like every other reference here.
 */

/* Nearest bf16 value to a double, ties to even, returned as a double (no
 * detour through binary32, which would round twice).  bf16 keeps 8
 * significant bits with binary32's exponent range: normal numbers are
 * rounded at 2^(e-7) for |x| in [2^e, 2^(e+1)); below 2^-126 the step is the
 * fixed subnormal quantum 2^-133.  Values that round beyond the largest
 * finite bf16, (2 - 2^-7) * 2^127, become infinities. */
static double round_bf16_d(double x)
{
    if (x != x || x == 0.0) return x;
    const double ax = fabs(x);
    if (ax == INFINITY) return x;
    double step;
    if (ax < ldexp(1.0, -126)) {
        step = ldexp(1.0, -133);
    } else {
        int e;
        (void)frexp(ax, &e);            /* ax in [2^(e-1), 2^e) */
        step = ldexp(1.0, e - 1 - 7);
    }
    const double r = nearbyint(x / step) * step;   /* exact scaling; ties to even */
    if (fabs(r) > ldexp(2.0 - ldexp(1.0, -7), 127)) return x > 0 ? INFINITY : -INFINITY;
    return r;
}

double oracle_round_bf16_d(double x) { return round_bf16_d(x); }

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^-x). */
static double silu(double x) { return x / (1.0 + exp(-x)); }

double oracle_silu(double x) { return silu(x); }

void oracle_round_bf16_d_array(int64_t n, const double *x, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = round_bf16_d(x[i]);
}

void oracle_silu_array(int64_t n, const double *x, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = silu(x[i]);
}

/* Y[i][j] = SiLU(round_bf16(sum_k A[i][k] B[k][j])), bf16 inputs, double out. */
void oracle_gemm_bf16_silu(int64_t M, int64_t N, int64_t K,
                           const uint16_t *A, int64_t lda,
                           const uint16_t *B, int64_t ldb,
                           double *Y, int64_t ldy)
{
    oracle_gemm_f64_from_bf16(M, N, K, A, lda, B, ldb, Y, ldy);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) Y[i * ldy + j] = silu(round_bf16_d(Y[i * ldy + j]));
}

/* SwiGLU on a merged gate/up weight: Wgu is [K][2N] with W_g in columns
 * 0..N-1 and W_u in columns N..2N-1.  With G and U the double products,
 * g = round_bf16(G), u = round_bf16(U), t = round_bf16(SiLU(g)) and
 * Z = t * u (unrounded).  g, u and t are returned too ([M][N], ldz). */
/* The activation chain of page "Operator & Runtime" §5.3.1 on stored bf16
 * G and U (Example 5-4), element by element: t = bf16(SiLU(g)) -- the value
 * the separate SiLU step stores -- and z = t * u, returned unrounded (the
 * product step stores bf16(z)). */
void oracle_silu_mul_bf16(int64_t n, const uint16_t *G, const uint16_t *U, double *t, double *z)
{
    for (int64_t i = 0; i < n; ++i) {
        t[i] = round_bf16_d(silu(widen_bf16(G[i])));
        z[i] = t[i] * widen_bf16(U[i]);
    }
}

void oracle_swiglu_bf16(int64_t M, int64_t N, int64_t K,
                        const uint16_t *X, int64_t ldx,
                        const uint16_t *Wgu, int64_t ldw,
                        double *Z, double *g, double *u, double *t, int64_t ldz)
{
    oracle_gemm_f64_from_bf16(M, N, K, X, ldx, Wgu, ldw, g, ldz);
    oracle_gemm_f64_from_bf16(M, N, K, X, ldx, Wgu + N, ldw, u, ldz);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            const int64_t o = i * ldz + j;
            g[o] = round_bf16_d(g[o]);
            u[o] = round_bf16_d(u[o]);
            t[o] = round_bf16_d(silu(g[o]));
            Z[o] = t[o] * u[o];
        }
}

/* ---------------------------------------------------------------------
 * The affine epilogue of a bf16 product: C := alpha * (A.B) + bias[j] +
 * beta * C_old[i][j], the product accumulated exactly (double), every term
 * widened exactly to double (bias and a bf16 C_old from their bf16 bit
 * patterns), returned unrounded.  bias may be NULL (no bias); C_old is read
 * only when beta != 0.  c_old_f32 selects float (1) or bf16 (0) C_old.
 */
void oracle_gemm_bf16_affine(int64_t M, int64_t N, int64_t K,
                             const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                             double alpha, const uint16_t *bias, double beta,
                             const void *C_old, int64_t ldc_old, int c_old_f32,
                             double *C, int64_t ldc)
{
    oracle_gemm_f64_from_bf16(M, N, K, A, lda, B, ldb, C, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * C[i * ldc + j];
            if (bias) v += widen_bf16(bias[j]);
            if (beta != 0.0) {
                const double old = c_old_f32 ? (double)((const float *)C_old)[i * ldc_old + j]
                                             : widen_bf16(((const uint16_t *)C_old)[i * ldc_old + j]);
                v += beta * old;
            }
            C[i * ldc + j] = v;
        }
}

/* ---------------------------------------------------------------------
 * FP8 quantization and the scaled FP8 product ("Operator & Runtime", §5.4.3,
 * Example 5-7 and Example 5-8).
 *
 * E4M3FN, as the page states it: an 8-bit float with 1 sign bit, 4 exponent
 * bits and 3 mantissa bits, largest finite value 448.  With exponent bias 7
 * a code s eeee mmm is (-1)^s (1 + m/8) 2^(e-7) for e >= 1; e = 0 holds the
 * subnormals (-1)^s m 2^-9; there are no infinities, and e = 15 with m = 7
 * is NaN (so 448 = 1.75 * 2^8 is the largest finite value).
 *
 * Per-row quantization with a scale from the whole row's maximum (Example
 * 5-7: the row is read first, then quantized): for a row x with
 * amax = max |x|, each element becomes the nearest E4M3FN value of
 * x * 448 / amax and dequantizes by the factor amax / 448.  The decision
 * that picks a code is taken in binary32, the kernel's precision:
 * inv = fl(448 / amax), y = fl(x * inv), y clamped to [-448, 448], then
 * rounded to the nearest E4M3FN value, ties to the code with the even
 * mantissa.  The dequantization factor is fl(amax / 448).  A row of zeros
 * has amax = 0, inv = 0, codes 0 and factor 0.
 */
static double e4m3_decode(uint8_t c)
{
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (c & 0x80) ? -v : v;
}

/* Nearest E4M3FN code to x (NaN -> 0x7f, |x| > 448 saturates to +-448). */
static uint8_t e4m3_encode(double x)
{
    if (x != x) return 0x7f;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a > 448.0) a = 448.0;
    /* spacing of representable values around a: 2^-9 below 2^-6 (the
     * subnormals and the first binade share it), else 2^(E-3) for a in
     * [2^E, 2^(E+1)) */
    double step;
    if (a < ldexp(1.0, -6)) {
        step = ldexp(1.0, -9);
    } else {
        int ex;
        (void)frexp(a, &ex);               /* a in [2^(ex-1), 2^ex) */
        step = ldexp(1.0, ex - 1 - 3);
    }
    /* a / step is exact (power-of-two scaling); nearbyint rounds half to
     * even, and an even multiple of the step is an even mantissa */
    const double q = nearbyint(a / step) * step;
    if (q == 0.0) return sign;
    if (q < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(q / ldexp(1.0, -9)));
    int ex;
    const double f = frexp(q, &ex);          /* q = f 2^ex, f in [0.5, 1) */
    const int e = ex - 1 + 7;
    const int m = (int)((2.0 * f - 1.0) * 8.0);
    return (uint8_t)(sign | (e << 3) | m);
}

double oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t oracle_e4m3_encode(double x) { return e4m3_encode(x); }

void oracle_e4m3_encode_array(int64_t n, const double *x, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}

/* Nearest binary32 value of x (ties to even), overflow to +-infinity: the
 * rounding of one binary32 operation whose exact result is x. */
static float rn_f32(double x)
{
    if (x != x) return (float)x;
    /* 2^128 - 2^103 is the midpoint between FLT_MAX and 2^128; from there on
     * binary32 rounding overflows */
    if (fabs(x) >= ldexp(1.0, 128) - ldexp(1.0, 103)) return x > 0 ? INFINITY : -INFINITY;
    return (float)x;
}

/* Fixed-range E4M3FN quantization, page "Operator & Runtime" §5.3.1
 * (Example 5-4 carried on: Z is stored with one fixed scale factor, one byte
 * per element).  The range amax (finite, > 0) maps to the format's largest
 * finite value 448, as in the per-row quantizer of §5.4.3, and the factor
 * that undoes it is amax / 448.  The page leaves the precision of that
 * quotient open; it is taken in binary32: z = fl(v), p = fl(z * 448),
 * y = fl(p / amax), each correctly rounded, and the code is the E4M3FN value
 * nearest to y (ties to the even mantissa, beyond +-448 saturating to
 * +-448, NaN to 0x7f).  The double quotient rounded to binary32 equals the
 * binary32 quotient (53 >= 2 * 24 + 2: rounding twice is innocuous for a
 * division).  What is quantized is the value the unfused program stores:
 * for SwiGLU the bf16 Z (§5.4.3 keeps the unfused program's roundings when
 * steps are fused), so v holds bf16 values there and fl(v), fl(z * 448)
 * are exact. */
void oracle_quantize_fixed_e4m3(int64_t n, const double *v, float amax, uint8_t *out)
{
    /* (amax finite and > 0: the Python wrapper checks it) */
    for (int64_t i = 0; i < n; ++i) {
        const float z = rn_f32(v[i]);
        const float p = rn_f32((double)z * 448.0);
        const float y = rn_f32((double)p / (double)amax);
        out[i] = e4m3_encode((double)y);
    }
}

/* Per-row E4M3FN quantization of bf16 rows X [rows, cols] into codes Q
 * (row stride ldq) and dequantization factors scale[rows], as page
 * "Operator & Runtime" defines it (§5.4.3, Example 5-7): the row's largest
 * magnitude amax maps to the format's largest finite value 448, so an
 * element x becomes the E4M3FN value nearest to the exact quotient
 * x * 448 / amax (ties to the even mantissa), and the factor that undoes it
 * is amax / 448.
 *
 * The code is decided exactly, with no rounded quotient: |x| * 448 and
 * v * amax, for v an E4M3FN value or the midpoint of two neighbours, are
 * products of at most 8 and 5 significant bits, exact in binary64, so
 * "x * 448 / amax < v" is decided by comparing |x| * 448 with v * amax.
 * The magnitude code is the number of positive E4M3FN values whose midpoint
 * with their successor lies below the quotient (binary search over the 126
 * midpoints), with a quotient exactly on a midpoint going to the
 * neighbour whose code is even.  |x| <= amax keeps the quotient at or
 * below 448.  The factor is amax / 448 rounded once to binary32 (the
 * division in binary64 cannot land on a binary32 midpoint: amax / 7 has a
 * periodic binary expansion).  A row of zeros gives codes 0 and factor 0;
 * a NaN element gives the NaN code. */
void oracle_quantize_rows_e4m3(int64_t rows, int64_t cols, const uint16_t *X, int64_t ldx,
                               uint8_t *Q, int64_t ldq, float *scale)
{
    /* mid[c] = (value(c) + value(c + 1)) / 2 for the magnitude codes
     * c = 0 .. 125 (value(126) = 448 is the largest finite) */
    double mid[126];
    for (int c = 0; c < 126; ++c) mid[c] = 0.5 * (e4m3_decode((uint8_t)c) + e4m3_decode((uint8_t)(c + 1)));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *x = X + r * ldx;
        double amax = 0.0;
        for (int64_t k = 0; k < cols; ++k) {
            const double v = fabs(widen_bf16(x[k]));
            if (v > amax) amax = v;
        }
        scale[r] = (float)(amax / 448.0);
        for (int64_t k = 0; k < cols; ++k) {
            const double v = widen_bf16(x[k]);
            if (v != v) {
                Q[r * ldq + k] = 0x7f;
                continue;
            }
            const uint8_t sign = signbit(v) ? 0x80 : 0x00;
            if (amax == 0.0) {
                Q[r * ldq + k] = sign;
                continue;
            }
            const double num = fabs(v) * 448.0;          /* exact */
            /* lo = number of midpoints strictly below the quotient */
            int lo = 0, hi = 126;
            while (lo < hi) {
                const int m = (lo + hi) / 2;
                if (mid[m] * amax < num) lo = m + 1;     /* both sides exact */
                else hi = m;
            }
            int c = lo;                                  /* nearest from above the midpoints below */
            if (c < 126 && mid[c] * amax == num && (c & 1)) c += 1;   /* tie: even neighbour */
            Q[r * ldq + k] = (uint8_t)(sign | c);
        }
    }
}

/* The scaled FP8 product with B given transposed (Bt [N, K]):
 * C[i][j] = (sum_k dec(A[i][k]) dec(Bt[j][k])) * sa[i] * sb[j], in double,
 * k ascending; a NULL scale vector means factors of 1.  The products of two
 * E4M3FN values (4 significant bits each) and their sums are exact in
 * double at these sizes. */
void oracle_gemm_fp8_nt(int64_t M, int64_t N, int64_t K,
                        const uint8_t *A, int64_t lda, const float *sa,
                        const uint8_t *Bt, int64_t ldb, const float *sb,
                        double *C, int64_t ldc)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += e4m3_decode(A[i * lda + k]) * e4m3_decode(Bt[j * ldb + k]);
            if (sa) acc *= (double)sa[i];
            if (sb) acc *= (double)sb[j];
            C[i * ldc + j] = acc;
        }
}

/* The scaled FP8 product followed by the affine epilogue of the bf16 path:
 * C = alpha * D + bias[j] + beta * C_old[i][j] with D as oracle_gemm_fp8_nt
 * computes it, in double (bias and a bf16 C_old widened exactly). */
void oracle_gemm_fp8_nt_affine(int64_t M, int64_t N, int64_t K,
                               const uint8_t *A, int64_t lda, const float *sa,
                               const uint8_t *Bt, int64_t ldb, const float *sb,
                               double alpha, const uint16_t *bias, double beta,
                               const void *C_old, int64_t ldc_old, int c_old_f32,
                               double *C, int64_t ldc)
{
    oracle_gemm_fp8_nt(M, N, K, A, lda, sa, Bt, ldb, sb, C, ldc);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * C[i * ldc + j];
            if (bias) v += widen_bf16(bias[j]);
            if (beta != 0.0) {
                const double old = c_old_f32 ? (double)((const float *)C_old)[i * ldc_old + j]
                                             : widen_bf16(((const uint16_t *)C_old)[i * ldc_old + j]);
                v += beta * old;
            }
            C[i * ldc + j] = v;
        }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the parallel loops above (timing the oracle on one core
 * and on all of them); no effect on any result. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
