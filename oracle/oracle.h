/*
 * oracle.h -- plain CPU reference for the mpgemm operations.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the package
 * entry file and the CPU-baseline leg of the benchmark may load this library.
 * The GPU library never links, includes or calls it, and it shares no code,
 * header, table or helper with the GPU library.
 *
 * Sources (the pages this oracle is written from):
 *  [L4]   "Hand-Written PTX Tensor-Core GEMM Kernels: A Multi-Precision Study on
 *         NVIDIA L4" -- the abstract (fugumt paper-check page) and the summary
 *         (thecoregrid page): dense GEMM in FP16, INT8 and INT4 arithmetic over
 *         square sizes N = 512 ... 8192.
 *  [SM75] "fused-int4-gemm-sm75" README -- project description and feature
 *         list: packed INT4 weights, sign extension, register dequantisation
 *         with per-group scales (group_size = 128), FP16 activations.
 *  [W4A4] "Warp-Specialized Kernel Implementation for W4A4 MatMul on Latest GPU
 *         Architectures", section 1 (Problem Definition): Y = Q(X) Q(W)^T, i.e.
 *         the weight operand is stored output-row major and enters transposed.
 *
 * Conventions shared with the GPU library only through the written contract
 * (C = A * B^T, B stored N x K, signed INT4 packed two per byte along K with the
 * low nibble holding the even k, symmetric per-(row, K-group) fp16 scales), not
 * through code.
 *
 * All functions are synchronous and parallelise over output rows with OpenMP;
 * per output element the arithmetic is the plain sequential k loop.
 */
#ifndef MPGEMM_ORACLE_H
#define MPGEMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_ARG = 1,      /* null pointer, negative size, ld too small, bad group */
    ORACLE_ERR_OVERFLOW = 2  /* an exact integer result does not fit int32 */
};

/* IEEE 754 binary16 bits -> the exact double value (subnormals, +-0, +-Inf, NaN). */
double oracle_f16_decode(uint16_t h);

/* double -> binary16 bits, round to nearest, ties to even; overflow -> +-Inf. */
uint16_t oracle_f16_encode_rne(double x);

/* Signed INT4 nibble k of a packed row: byte k/2, low nibble for even k. */
int oracle_i4_get(const uint8_t *row, int64_t k);

/* C[m*ldc+n] = sum_k A[m*lda+k] * B[n*ldb+k], exact (int64 accumulator).
 * [L4] abstract: INT8 arithmetic. Returns ORACLE_ERR_OVERFLOW (C fully written,
 * overflowing entries wrapped) if any exact sum leaves the int32 range. */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                   int32_t *C, int64_t ldc);

/* As oracle_gemm_i8 for signed INT4 operands packed two per byte along K.
 * lda and ldb count int4 elements (nibbles) and must be even; the byte stride
 * of a row is ld/2. [L4] summary INT4 paragraph; [SM75] "INT4 packing, sign
 * extension". */
int oracle_gemm_i4(int64_t M, int64_t N, int64_t K,
                   const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                   int32_t *C, int64_t ldc);

/* C[m*ldc+n] = sum_k a(m,k) * b(n,k) in double, k ascending, where a and b are
 * the binary16 inputs decoded exactly. [L4] abstract: FP16 arithmetic. */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                    double *C, int64_t ldc);

/* Weight-only INT4 GEMM ([SM75] feature list: register dequantisation,
 * per-group scales):
 *   Y[m*ldy+n] = sum_k x(m,k) * q(n,k) * s(n, k/G)      (double, k ascending)
 * X: M x K binary16, row stride ldx elements.
 * W: N x K signed INT4 packed along K, ldw counted in nibbles (even).
 * S: N x (K/G) binary16 scales, row stride lds elements.
 * T2 (optional, may be NULL): T2[m*ldt+n] = sum_k (x q s)^2, used by the tests
 * to size the tolerance for fp16 dequantisation.
 * Requires G >= 1 and K % G == 0. The output is the unrounded sum; the tests
 * round it with oracle_f16_encode_rne where the fp16 output is compared. */
int oracle_gemm_w4a16(int64_t M, int64_t N, int64_t K,
                      const uint16_t *X, int64_t ldx,
                      const uint8_t *W, int64_t ldw,
                      const uint16_t *S, int64_t lds, int64_t G,
                      double *Y, int64_t ldy, double *T2, int64_t ldt);

/* INT4 x INT4 GEMM with a scale epilogue ([W4A4] section 1: Y = (Q(X) Q(W)^T)
 * (.) scale + b, both operands 4-bit). Reading of the scale: one fp16 factor
 * per row of X (SX, M values) times one per row of W (SW, N values), applied to
 * the exact integer product; BIAS (N values, may be NULL) added per column:
 *   Y[m][n] = (sum_k qa(m,k) qb(n,k)) * SX[m] * SW[n] + BIAS[n]
 * in double, unrounded (the tests round to fp16 where they compare). A, B
 * packed as for oracle_gemm_i4. The low-rank branch L(X) is oracle_w4a4_lowrank. */
int oracle_gemm_w4a4(int64_t M, int64_t N, int64_t K,
                     const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                     const uint16_t *SX, const uint16_t *SW, const uint16_t *BIAS,
                     double *Y, int64_t ldy);

/* The low-rank residual branch L(X) of the W4A4 formula ("Warp-Specialized
 * Kernel Implementation for W4A4 MatMul on Latest GPU Architectures",
 * section 1: Y = (Q(X) Q(W)^T) (.) scale + L(X) + b; the page names a small
 * down- and up-projection pair and no precision, the reading used is):
 *   U[m][r] = sum_k X[m][k] LD[r][k]                (the unquantised fp16 input)
 *   L[m][n] = sum_r binary16_rne(U[m][r]) LU[n][r]  (U enters the second product as fp16)
 * X: M x K binary16 (row stride ldx), LD: R x K binary16 (the down-projection,
 * K-contiguous like a weight), LU: N x R binary16 (the up-projection, row
 * stride ldu). U (M x R) and L (M x N) in double, unrounded; U's sums are
 * double sums of exact products. The full W4A4 output is oracle_gemm_w4a4's
 * value plus L. */
int oracle_w4a4_lowrank(int64_t M, int64_t N, int64_t K, int64_t R,
                        const uint16_t *X, int64_t ldx, const uint16_t *LD, int64_t ldd,
                        const uint16_t *LU, int64_t ldu, double *U, int64_t ldU,
                        double *L, int64_t ldl);

/* Symmetric round-to-nearest INT4 quantisation of fp16 weights per
 * (row, G-wide K group), the step that produces the inputs of
 * oracle_gemm_w4a16 ([SM75] feature list: per-group scales, group_size = 128,
 * packed INT4 weights; the pages give no formula, the reading used is):
 *   s = binary16_rne(max_k |w| / 7)
 *   q = clamp(round_half_even(w / s), -8, 7), q = 0 when s == 0
 * W: N x K binary16 (row stride ldw elements); Q: packed like the GEMM's
 * weights (row stride ldq nibbles, even); S: N x K/G binary16 (row stride lds).
 * Requires K % G == 0 and K even. Inputs must be finite. */
int oracle_quantize_w4(int64_t N, int64_t K, const uint16_t *W, int64_t ldw, int64_t G,
                       uint8_t *Q, int64_t ldq, uint16_t *S, int64_t lds);

/* Number of OpenMP threads a call uses. */
int oracle_threads(void);
/* Threads of the next oracle calls (n > 0; for single-thread timings). */
void oracle_set_threads(int n);

#ifdef __cplusplus
}
#endif

#endif
