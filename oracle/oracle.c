/*
 * oracle.c -- plain CPU reference for the mpgemm operations.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing). It is
 * deliberately slow and literal: every result is the textbook definition of
 * the operation written out as a loop over k, with no blocking, no fusion and
 * no reordering. See oracle.h for the sources each function follows.
 *
 * Built with gcc -O2 -fopenmp (no fast-math, so double sums keep their
 * sequential k order). OpenMP splits only the loop over output rows.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- binary16 */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0: subnormal, value = f * 2^-24; exponent 31: Inf (f == 0) or NaN;
 * otherwise value = (1024 + f) * 2^(e - 25). */
double oracle_f16_decode(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* Round to nearest, ties to even. The magnitude is scaled by a power of two so
 * that the retained significand is an integer (exact), and nearbyint() rounds
 * it in the default FE_TONEAREST mode, which is round-half-to-even. */
uint16_t oracle_f16_encode_rne(double x)
{
    if (isnan(x))
        return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* 65504 is the largest finite binary16; the midpoint to 2^16 is 65520 and
     * ties go to the even neighbour 2^16, which is Inf. */
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; q == 1024 is the smallest normal,
         * whose bit pattern is exactly 1024. */
        double q = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    int ex;
    (void)frexp(a, &ex);             /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                  /* a in [2^e, 2^(e+1)) */
    double q = nearbyint(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

/* -------------------------------------------------------------------- int4 */

/* Signed INT4 element k of a packed row: byte k/2, low nibble for even k and
 * high nibble for odd k, two's complement in [-8, 7]. */
int oracle_i4_get(const uint8_t *row, int64_t k)
{
    int byte = row[k / 2];
    int v = (k % 2 == 0) ? (byte & 0xF) : ((byte >> 4) & 0xF);
    return (v >= 8) ? v - 16 : v;
}

/* -------------------------------------------------------------------- gemm */

static int check_dims(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                      const void *A, const void *B, const void *C)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_ERR_ARG;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    if (!C || (K > 0 && (!A || !B)))
        return ORACLE_ERR_ARG;
    if (lda < K || ldb < K || ldc < N)
        return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                   int32_t *C, int64_t ldc)
{
    int st = check_dims(M, N, K, lda, ldb, ldc, A, B, C);
    if (st != ORACLE_OK || M == 0 || N == 0)
        return st;
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)A[m * lda + k] * (int64_t)B[n * ldb + k];
            if (acc > INT32_MAX || acc < INT32_MIN)
                overflow = 1;
            C[m * ldc + n] = (int32_t)(uint32_t)acc;
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

int oracle_gemm_i4(int64_t M, int64_t N, int64_t K,
                   const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                   int32_t *C, int64_t ldc)
{
    if ((lda % 2) != 0 || (ldb % 2) != 0)
        return ORACLE_ERR_ARG;
    int st = check_dims(M, N, K, lda, ldb, ldc, A, B, C);
    if (st != ORACLE_OK || M == 0 || N == 0)
        return st;
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t *arow = A + m * (lda / 2);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *brow = B + n * (ldb / 2);
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)oracle_i4_get(arow, k) * (int64_t)oracle_i4_get(brow, k);
            if (acc > INT32_MAX || acc < INT32_MIN)
                overflow = 1;
            C[m * ldc + n] = (int32_t)(uint32_t)acc;
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* Decode a rows x K block of binary16 values (row stride ld) into a dense
 * rows x K double array. Returns NULL on allocation failure. */
static double *decode_rows(const uint16_t *P, int64_t rows, int64_t K, int64_t ld)
{
    size_t count = (size_t)rows * (size_t)(K > 0 ? K : 1);
    double *D = (double *)malloc(count * sizeof(double));
    if (!D)
        return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            D[r * K + k] = oracle_f16_decode(P[r * ld + k]);
    return D;
}

int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                    double *C, int64_t ldc)
{
    int st = check_dims(M, N, K, lda, ldb, ldc, A, B, C);
    if (st != ORACLE_OK || M == 0 || N == 0)
        return st;
    double *a = decode_rows(A, M, K, lda);
    double *b = decode_rows(B, N, K, ldb);
    if (!a || !b) {
        free(a);
        free(b);
        return ORACLE_ERR_ARG;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += a[m * K + k] * b[n * K + k];
            C[m * ldc + n] = acc;
        }
    }
    free(a);
    free(b);
    return ORACLE_OK;
}

int oracle_gemm_w4a16(int64_t M, int64_t N, int64_t K,
                      const uint16_t *X, int64_t ldx,
                      const uint8_t *W, int64_t ldw,
                      const uint16_t *S, int64_t lds, int64_t G,
                      double *Y, int64_t ldy, double *T2, int64_t ldt)
{
    if (G < 1 || (K % G) != 0 || (ldw % 2) != 0)
        return ORACLE_ERR_ARG;
    int st = check_dims(M, N, K, ldx, ldw, ldy, X, W, Y);
    if (st != ORACLE_OK || M == 0 || N == 0)
        return st;
    if (K > 0 && (!S || lds < K / G))
        return ORACLE_ERR_ARG;
    if (T2 && ldt < N)
        return ORACLE_ERR_ARG;
    double *x = decode_rows(X, M, K, ldx);
    if (!x)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *wrow = W + n * (ldw / 2);
            double acc = 0.0, sq = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double s = oracle_f16_decode(S[n * lds + k / G]);
                double t = x[m * K + k] * (double)oracle_i4_get(wrow, k) * s;
                acc += t;
                sq += t * t;
            }
            Y[m * ldy + n] = acc;
            if (T2)
                T2[m * ldt + n] = sq;
        }
    }
    free(x);
    return ORACLE_OK;
}

int oracle_gemm_w4a4(int64_t M, int64_t N, int64_t K,
                     const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                     const uint16_t *SX, const uint16_t *SW, const uint16_t *BIAS,
                     double *Y, int64_t ldy)
{
    if ((K % 2) != 0 || (lda % 2) != 0 || (ldb % 2) != 0)
        return ORACLE_ERR_ARG;
    int st = check_dims(M, N, K, lda, ldb, ldy, A, B, Y);
    if (st != ORACLE_OK || M == 0 || N == 0)
        return st;
    if (!SX || !SW)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t *arow = A + m * (lda / 2);
        const double sx = oracle_f16_decode(SX[m]);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *brow = B + n * (ldb / 2);
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)oracle_i4_get(arow, k) * (int64_t)oracle_i4_get(brow, k);
            double y = (double)acc * sx * oracle_f16_decode(SW[n]);
            if (BIAS)
                y += oracle_f16_decode(BIAS[n]);
            Y[m * ldy + n] = y;
        }
    }
    return ORACLE_OK;
}

int oracle_w4a4_lowrank(int64_t M, int64_t N, int64_t K, int64_t R,
                        const uint16_t *X, int64_t ldx, const uint16_t *LD, int64_t ldd,
                        const uint16_t *LU, int64_t ldu, double *U, int64_t ldU,
                        double *L, int64_t ldl)
{
    if (M < 0 || N < 0 || K < 0 || R < 0)
        return ORACLE_ERR_ARG;
    if (M == 0 || N == 0 || R == 0)
        return ORACLE_OK;
    if (!X || !LD || !LU || !U || !L || ldx < K || ldd < K || ldu < R || ldU < R || ldl < N)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        /* step 1: the down-projection of the row, U[m][r] = sum_k X[m][k] LD[r][k] */
        for (int64_t r = 0; r < R; ++r) {
            double u = 0.0;
            for (int64_t k = 0; k < K; ++k)
                u += oracle_f16_decode(X[m * ldx + k]) * oracle_f16_decode(LD[r * ldd + k]);
            U[m * ldU + r] = u;
        }
        /* step 2: the up-projection of U rounded to binary16 (nearest even) */
        for (int64_t n = 0; n < N; ++n) {
            double l = 0.0;
            for (int64_t r = 0; r < R; ++r)
                l += oracle_f16_decode(oracle_f16_encode_rne(U[m * ldU + r])) * oracle_f16_decode(LU[n * ldu + r]);
            L[m * ldl + n] = l;
        }
    }
    return ORACLE_OK;
}

int oracle_quantize_w4(int64_t N, int64_t K, const uint16_t *W, int64_t ldw, int64_t G,
                       uint8_t *Q, int64_t ldq, uint16_t *S, int64_t lds)
{
    if (N < 0 || K < 0 || G < 1 || (K % G) != 0 || (K % 2) != 0 || (ldq % 2) != 0)
        return ORACLE_ERR_ARG;
    if (N == 0 || K == 0)
        return ORACLE_OK;
    if (!W || !Q || !S || ldw < K || ldq < K || lds < K / G)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *qrow = Q + n * (ldq / 2);
        for (int64_t k = 0; k < K / 2; ++k)
            qrow[k] = 0;
        for (int64_t g = 0; g < K / G; ++g) {
            /* step 1: the group's largest magnitude */
            double amax = 0.0;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                double a = fabs(oracle_f16_decode(W[n * ldw + k]));
                if (a > amax)
                    amax = a;
            }
            /* step 2: the scale, amax / 7 rounded to binary16 */
            uint16_t sbits = oracle_f16_encode_rne(amax / 7.0);
            double s = oracle_f16_decode(sbits);
            S[n * lds + g] = sbits;
            /* step 3: each weight divided by the stored scale, rounded to the
               nearest integer (ties to even), clamped to the signed 4-bit range */
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                int q = 0;
                if (s > 0.0) {
                    double r = nearbyint(oracle_f16_decode(W[n * ldw + k]) / s);
                    q = r > 7.0 ? 7 : (r < -8.0 ? -8 : (int)r);
                }
                const uint8_t nib = (uint8_t)(q & 0xF);
                qrow[k / 2] |= (uint8_t)((k % 2) ? (nib << 4) : nib);
            }
        }
    }
    return ORACLE_OK;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
