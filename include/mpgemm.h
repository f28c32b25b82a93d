/*
 * mpgemm.h -- multi-precision dense GEMM for AMD Instinct MI355X (gfx950).
 *
 * Operations (all compute C = A * B^T with A of M x K and B of N x K, both
 * row-major and K-contiguous, C row-major M x N, alpha = 1, beta = 0):
 *
 *   mpgemm_run_f16    fp16 x fp16, fp32 accumulate, fp32 C
 *   mpgemm_run_i8     int8 x int8, int32 accumulate, int32 C (exact)
 *   mpgemm_run_i4     signed int4 x signed int4 packed two per byte along K,
 *                     int32 accumulate, int32 C (exact)
 *   mpgemm_run_w4a16  fp16 activations x int4 weights with per-(row, K-group)
 *                     fp16 scales, fp32 accumulate, fp16 Y
 *   mpgemm_run_w4a4   int4 x int4 with per-row and per-column fp16 scales and
 *                     a column bias applied to the exact int32 sum, fp16 Y
 *   mpgemm_run_{f16,i8,i4}_kn  the first three with B stored K x N (the
 *                     transposed layout, kept as a measured control)
 *
 * Sources: "Hand-Written PTX Tensor-Core GEMM Kernels: A Multi-Precision Study
 * on NVIDIA L4" (abstract and summary: the FP16 / INT8 / INT4 GEMM problem over
 * square sizes N = 512 ... 8192) and the "fused-int4-gemm-sm75" README (project
 * description and feature list: packed INT4 weights, sign extension, in-register
 * dequantisation with per-group scales, group_size = 128, FP16 activations,
 * M = 1 decode and M = 128 prefill at 4096 x 4096). The weight operand enters
 * transposed as in Y = Q(X) Q(W)^T of "Warp-Specialized Kernel Implementation
 * for W4A4 MatMul on Latest GPU Architectures", section 1.
 *
 * Common contract of every run call
 * ---------------------------------
 *  - Pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or retains them. Buffers must stay valid until the work
 *    queued on `stream` has finished.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous: they validate, enqueue kernels and return. A fault inside
 *    a kernel is reported by the caller's next synchronisation, not here.
 *  - Leading dimensions count elements of the logical type (for packed INT4:
 *    nibbles, which must be even; the byte stride of a row is ld / 2).
 *    Required: lda >= K, ldb >= K, ldc >= N.
 *  - Alignment: outputs need only the alignment of their element type. For
 *    mpgemm_run_{f16,i8,i4}, A and B may have any alignment, but rows that are
 *    16-byte aligned (base pointer and row stride in bytes) take the fast
 *    kernel; other rows are read with byte gathers. mpgemm_run_w4a16 requires
 *    X and Wq 16-byte aligned with row strides that are multiples of 16 bytes
 *    (else MPGEMM_ERR_UNSUPPORTED); S and Y need 2-byte alignment.
 *  - M == 0 or N == 0 is a no-op returning MPGEMM_OK. K == 0 writes zeros.
 *  - Only the first K elements of each input row enter the result, and only
 *    the first N elements of each output row are written. The fast kernel
 *    may read (and discard) the bytes of a row up to its next 16-byte
 *    boundary; such a read never crosses into another page.
 *  - Argument errors return before any HIP call and leave outputs untouched.
 *  - Output rows may not overlap inputs.
 *  - A handle owns 128 MiB + 64 KiB of device memory, allocated by
 *    mpgemm_create and freed by mpgemm_destroy: the workspace where
 *    mpgemm_run_w4a16 keeps the fp32 partial sums of a K split and where a
 *    stream-K launch of mpgemm_run_{f16,i8,i4,w4a4} keeps partial tiles and
 *    its per-tile arrival counters. No call allocates memory.
 *  - Calls that share a handle must not overlap in time (issue them on one
 *    stream, or use one handle per stream): they share its workspace. A
 *    stream-K launch leaves its counters at zero when it completes; a launch
 *    that never completes (a fault) leaves the handle unusable.
 *  - Results do not depend on the schedule: stream-K partial tiles are summed
 *    in a fixed order, so repeated calls give bit-identical outputs.
 */
#ifndef MPGEMM_H
#define MPGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mpgemm_ctx *mpgemm_handle_t;

typedef enum {
    MPGEMM_OK = 0,
    MPGEMM_ERR_INVALID_ARG = 1,  /* null handle/pointer, negative size, ld too small */
    MPGEMM_ERR_UNSUPPORTED = 2,  /* alignment, odd K or ld for INT4, group size, K bound */
    MPGEMM_ERR_DEVICE = 3,       /* no GPU, or the device is not gfx950 */
    MPGEMM_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} mpgemm_status_t;

/* Create a handle bound to `device` (device < 0: the current device). Checks
 * that the device exists and is gfx950, caches its compute-unit count and
 * allocates the handle's workspace (MPGEMM_ERR_HIP if that fails). */
mpgemm_status_t mpgemm_create(mpgemm_handle_t *out, int device);

/* Destroy a handle. NULL is accepted (no-op). */
mpgemm_status_t mpgemm_destroy(mpgemm_handle_t h);

/* Static, human-readable name of a status code. */
const char *mpgemm_status_string(mpgemm_status_t s);

/* Largest K accepted by the integer paths: every exact sum stays in int32
 * (128 * 128 * K < 2^31 for INT8, and the INT4 kernel's 16x-scaled operands
 * have the same bound). */
#define MPGEMM_MAX_K_INT 131071

/* FP16 GEMM ([L4 study] abstract: FP16 arithmetic).
 * A: M x K binary16 (row stride lda), B: N x K binary16 (row stride ldb),
 * C: M x N float (row stride ldc). C[m][n] = sum_k A[m][k] * B[n][k], every
 * product and partial sum in fp32 (IEEE round to nearest); the summation
 * order is unspecified. */
mpgemm_status_t mpgemm_run_f16(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda,
                               const uint16_t *B, int64_t ldb,
                               float *C, int64_t ldc, void *stream);

/* INT8 GEMM ([L4 study] abstract and INT8 paragraph of the summary).
 * A: M x K int8, B: N x K int8, C: M x N int32, exact.
 * K <= MPGEMM_MAX_K_INT, else MPGEMM_ERR_UNSUPPORTED. */
mpgemm_status_t mpgemm_run_i8(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                              const int8_t *A, int64_t lda,
                              const int8_t *B, int64_t ldb,
                              int32_t *C, int64_t ldc, void *stream);

/* INT4 GEMM ([L4 study] abstract and INT4 paragraph of the summary).
 * A: M x K signed INT4 packed two per byte along K: byte k/2 of a row holds
 * element k in its low nibble when k is even and in its high nibble when k is
 * odd, two's complement in [-8, 7]. B: N x K, same format. C: M x N int32,
 * exact. K, lda and ldb must be even (nibble counts); K <= MPGEMM_MAX_K_INT. */
mpgemm_status_t mpgemm_run_i4(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                              const uint8_t *A, int64_t lda,
                              const uint8_t *B, int64_t ldb,
                              int32_t *C, int64_t ldc, void *stream);

/* Transposed-B layout: the control of the [L4 study] summary's ablation of
 * the B operand's layout (the INT4 k64 paragraph: a transposed B is the
 * worse layout). The same products as mpgemm_run_{f16,i8,i4}, with B stored
 * K x N: C[m][n] = sum_k A[m][k] * Bt[k][n], Bt row-major with row stride
 * ldbt >= N elements. A is M x K as above. For INT4 the elements of a Bt row
 * are packed two per byte along n (byte n/2 of row k holds n in its low
 * nibble when n is even); K, lda and ldbt must be even; N may be odd (the
 * high nibble of a row's last byte is then ignored).
 * These calls exist to measure that layout and have one kernel only: A and Bt
 * must be 16-byte aligned with row strides that are multiples of 16 bytes,
 * else MPGEMM_ERR_UNSUPPORTED. Everything else (ownership, errors, no-ops, K
 * bound for the integer paths, accumulation) is as for the N x K calls. */
mpgemm_status_t mpgemm_run_f16_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                  const uint16_t *A, int64_t lda,
                                  const uint16_t *Bt, int64_t ldbt,
                                  float *C, int64_t ldc, void *stream);
mpgemm_status_t mpgemm_run_i8_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const int8_t *A, int64_t lda,
                                 const int8_t *Bt, int64_t ldbt,
                                 int32_t *C, int64_t ldc, void *stream);
mpgemm_status_t mpgemm_run_i4_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const uint8_t *A, int64_t lda,
                                 const uint8_t *Bt, int64_t ldbt,
                                 int32_t *C, int64_t ldc, void *stream);

/* INT4 x INT4 GEMM with a scale epilogue ("Warp-Specialized Kernel
 * Implementation for W4A4 MatMul on Latest GPU Architectures", section 1:
 * Y = (Q(X) Q(W)^T) (.) scale + b with 4-bit activations and weights; the
 * page gives no scale layout, the reading used is one factor per activation
 * row and one per weight row, applied to the exact integer product, and a
 * bias per output column; the low-rank branch L(X) is left to the next call):
 *   Y[m][n] = fp16( (sum_k qa(m, k) qb(n, k)) * SX[m] * SW[n] + bias[n] )
 * A, B: packed signed INT4 exactly as for mpgemm_run_i4 (K, lda, ldb even,
 * K <= MPGEMM_MAX_K_INT). SX: M binary16, SW: N binary16, bias: N binary16 or
 * NULL (no bias); all 2-byte aligned. Y: M x N binary16, row stride ldy.
 * The integer sum is exact; the two products and the bias are applied in
 * fp32 (each correctly rounded), then one rounding to fp16 (nearest even).
 * The low-rank branch L(X) is mpgemm_run_w4a4_lowrank. */
mpgemm_status_t mpgemm_run_w4a4(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                const uint8_t *A, int64_t lda,
                                const uint8_t *B, int64_t ldb,
                                const uint16_t *SX, const uint16_t *SW, const uint16_t *bias,
                                uint16_t *Y, int64_t ldy, void *stream);

/* W4A4 with the formula's low-rank residual branch ("Warp-Specialized Kernel
 * Implementation for W4A4 MatMul on Latest GPU Architectures", section 1:
 * Y = (Q(X) Q(W)^T) (.) scale + L(X) + b, L a small down- and up-projection
 * of the unquantised input; the page fixes no precision, the reading used is
 * fp16 operands with fp32 sums and the projected activations rounded to fp16
 * before the up-projection):
 *   U[m][r] = sum_k X[m][k] LD[r][k]                        (fp32 sum)
 *   L[m][n] = sum_r fp16_rne(U[m][r]) LU[n][r]               (fp32 sum)
 *   Y[m][n] = fp16( (((sum_k qa qb) * SX[m]) * SW[n] + L[m][n]) + bias[n] )
 * A, B, SX, SW, bias, Y: exactly as for mpgemm_run_w4a4.
 * X:  M x K binary16, the unquantised activations, row stride ldx >= K.
 * LD: R x K binary16, the down-projection (K-contiguous), row stride ldd >= K.
 * LU: N x R binary16, the up-projection (R-contiguous), row stride ldu >= R.
 * R must be a multiple of 16 with R <= MPGEMM_MAX_LOWRANK, LU 16-byte aligned
 * with ldu a multiple of 8, X and LD 2-byte aligned (else
 * MPGEMM_ERR_UNSUPPORTED); R == 0 is mpgemm_run_w4a4. U lives in the
 * handle's workspace: M * R * 4 bytes (rounded up to 256) may take at most
 * half of it, else MPGEMM_ERR_UNSUPPORTED. Two launches on `stream`: U (by a
 * skinny down-projection kernel when R <= 64, K % 64 == 0 and X, LD have
 * 16-byte aligned rows, else by the FP16 tile kernel), then the W4A4 tile
 * kernel, whose epilogue adds L per 32 x 32 output block on the matrix unit.
 * The fp32 sums' order is unspecified; every other step rounds as written;
 * repeated calls give bit-identical results. */
#define MPGEMM_MAX_LOWRANK 256
mpgemm_status_t mpgemm_run_w4a4_lowrank(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                        const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                        const uint16_t *SX, const uint16_t *SW, const uint16_t *bias,
                                        const uint16_t *X, int64_t ldx, const uint16_t *LD, int64_t ldd,
                                        const uint16_t *LU, int64_t ldu, int64_t R,
                                        uint16_t *Y, int64_t ldy, void *stream);

/* Weight-only INT4 GEMM ("fused-int4-gemm-sm75" README: register
 * dequantisation, per-group scales with group_size = 128; decode M = 1 and
 * prefill M = 128).
 *   Y[m][n] = fp16_rne( sum_k X[m][k] * q(n, k) * S[n][k / G] )
 * X:  M x K binary16 activations, row stride ldx elements.
 * Wq: N x K signed INT4 weights packed along K exactly as for mpgemm_run_i4,
 *     row stride ldw nibbles (even).
 * S:  N x (K / G) binary16 scales, row stride lds elements (lds >= K / G).
 *     Symmetric quantisation: no zero point.
 * Y:  M x N binary16 output, row stride ldy elements, rounded to nearest even
 *     from the fp32 accumulator.
 * G must be a power of two with 32 <= G <= K and K % G == 0. The sum is
 * accumulated in fp32; where the scale is applied (to the fp16 weight before
 * the product, or to the fp32 group sum after it) is unspecified.
 * X and Wq are read with 16-byte loads (see the alignment rule above). */
mpgemm_status_t mpgemm_run_w4a16(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const uint16_t *X, int64_t ldx,
                                 const uint8_t *Wq, int64_t ldw,
                                 const uint16_t *S, int64_t lds, int64_t group_size,
                                 uint16_t *Y, int64_t ldy, void *stream);

/* Allocation-free weight-only INT4 GEMM, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. No handle: it runs on the caller's
 * current device, computes exactly what mpgemm_run_w4a16 computes with a
 * default handle (the same kernel plan, so bit-identical results), and takes
 * the same arguments with the same meaning, layout and checks.
 * The fp32 partial sums of a K split live in a static device array of
 * MPGEMM_NOALLOC_SCRATCH_BYTES per GPU (held by each GPU the library runs on
 * until the process ends); no call allocates or frees memory. A problem whose
 * split needs more than that returns MPGEMM_ERR_UNSUPPORTED before any
 * launch. Every call on one GPU shares that GPU's array, and each call
 * overwrites every partial sum it reads, so consecutive calls need no reset;
 * calls that overlap in time on one GPU (concurrent streams, or host
 * threads) race on the array and give undefined results: order them on one
 * stream. The first call on a device looks up that device's copy of the
 * array (MPGEMM_ERR_HIP if that fails); MPGEMM_ERR_DEVICE without a current
 * device. */
#define MPGEMM_NOALLOC_SCRATCH_BYTES (16 << 20)
mpgemm_status_t mpgemm_run_w4a16_noalloc(int64_t M, int64_t N, int64_t K,
                                         const uint16_t *X, int64_t ldx,
                                         const uint8_t *Wq, int64_t ldw,
                                         const uint16_t *S, int64_t lds, int64_t group_size,
                                         uint16_t *Y, int64_t ldy, void *stream);

/* Weight quantisation for mpgemm_run_w4a16 (the weights and scales it
 * consumes: "fused-int4-gemm-sm75" README, feature list: per-group scaling
 * factors, group_size = 128, packed INT4 weights; the README names no
 * formula, so the plainest symmetric round-to-nearest reading):
 *   S[n][g] = fp16_rne(max |W[n][k]| over k in group g, divided by 7)
 *   q(n, k) = clamp(round_half_even(W[n][k] / S[n][k / G]), -8, 7),
 *             q = 0 where the scale is 0
 * W:  N x K binary16 weights, row stride ldw elements; finite values.
 * Wq: N x K signed INT4 written packed exactly as mpgemm_run_w4a16 reads
 *     them, row stride ldwq nibbles (even); S: N x (K / G) binary16, row
 *     stride lds elements. G must be a power of two with 32 <= G <= 512 and
 *     K % G == 0 (else MPGEMM_ERR_UNSUPPORTED). W must be 16-byte aligned with
 *     a row stride that is a multiple of 16 bytes, Wq 4-byte aligned with a
 *     row stride that is a multiple of 4 bytes, S 2-byte aligned.
 * Results are bit-identical to the definition above in exact arithmetic. */
mpgemm_status_t mpgemm_quantize_w4(mpgemm_handle_t h, int64_t N, int64_t K,
                                   const uint16_t *W, int64_t ldw, int64_t group_size,
                                   uint8_t *Wq, int64_t ldwq, uint16_t *S, int64_t lds,
                                   void *stream);

/* Measurement aid: a plain streaming read of `bytes` bytes at `src` (device
 * memory, 16-byte aligned, bytes a multiple of 16) with 16-byte loads,
 * loads_per_lane (1, 2, 4 or 8) per lane, all issued before any is combined.
 * Workgroup b writes the XOR of every 32-bit word it read to sink[b]; the
 * XOR of sink[0 .. blocks) is the XOR of the whole buffer (blocks =
 * ceil(bytes / (4096 * loads_per_lane)), at most sink_words, else
 * MPGEMM_ERR_INVALID_ARG). It times the cold read of the bytes a memory-bound
 * call must move: the attainable ceiling measured on the card ("Warp-
 * Specialized Kernel Implementation for W4A4 MatMul on Latest GPU
 * Architectures", section 2: utilisation against a ceiling calibrated on the
 * same GPU). Asynchronous on `stream`; no handle. */
mpgemm_status_t mpgemm_stream_read(const void *src, int64_t bytes, int loads_per_lane,
                                   uint32_t *sink, int64_t sink_words, void *stream);

/* Precision tags of mpgemm_plan_gemm. */
enum {
    MPGEMM_PREC_F16 = 0,
    MPGEMM_PREC_I8 = 1,
    MPGEMM_PREC_I4 = 2,
    MPGEMM_PREC_W4A4 = 3
};

/* Planning queries: which kernel configuration a call with these sizes runs
 * on a device with cu_count compute units (with no configuration override),
 * decided on the host from the sizes alone; no device is touched.
 * mpgemm_plan_gemm: the tile configuration (the index the MPGEMM_TILE_CFG
 * override takes) of mpgemm_run_{f16,i8,i4,w4a4}; operands that are not
 * 16-byte aligned run the byte-gather kernel instead. sk_grid: 0 for a
 * data-parallel launch (one workgroup per output tile), else the number of
 * persistent workgroups of a stream-K launch, which runs the first
 * sk_tiles_dp tiles whole and splits the K loops of the remaining tiles
 * evenly over the grid (the MPGEMM_STREAMK=0/1 override turns it off, or on
 * whenever the tiles do not fill whole waves of the grid; =2 runs every tile
 * whole on a persistent grid of the resident workgroups, a measured
 * alternative).
 * mpgemm_plan_w4a16: the configuration of mpgemm_run_w4a16 (the index the
 * MPGEMM_W4A16_CFG override takes), the number of workgroups K is split over
 * (k_splits; 1 = no second reduction kernel) and the K extent of one split. */
mpgemm_status_t mpgemm_plan_gemm(int precision, int64_t M, int64_t N, int64_t K, int cu_count,
                                 int *config, int *sk_grid, int *sk_tiles_dp);
mpgemm_status_t mpgemm_plan_w4a16(int64_t M, int64_t N, int64_t K, int cu_count, int *config,
                                  int *k_splits, int64_t *k_slice);

#ifdef __cplusplus
}
#endif

#endif
