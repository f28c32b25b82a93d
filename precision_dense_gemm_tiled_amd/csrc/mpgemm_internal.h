// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mpgemm.h"

namespace mpg {

// PREC_W4A4: the INT4 main loop with a scale epilogue (fp16 output).
enum Prec { PREC_F16 = 0, PREC_I8 = 1, PREC_I4 = 2, PREC_W4A4 = 3 };

// One dense GEMM C = A * B^T, described in bytes of the packed K dimension:
// kbytes = 2K (f16), K (i8) or K/2 (i4). Row strides are in bytes for A and B
// and in output elements for C.
struct GemmProblem {
    const uint8_t *A;
    const uint8_t *B;
    void *C;
    int64_t lda_b, ldb_b, ldc;
    int M, N;
    int64_t kbytes;
    // PREC_W4A4 epilogue: C[m][n] = fp16(acc * sx[m] * sw[n] + bias[n]) (fp16
    // bits; bias may be null); unused by the other precisions
    const uint16_t *sx, *sw, *bias;
    // 1 when C and every C row start on a 16-byte boundary (the tile epilogue
    // may then store four consecutive 4-byte outputs at once)
    int c_vec16;
    // PREC_W4A4 low-rank branch, when lr_rank > 0 (a multiple of 16): the
    // epilogue adds sum_r fp16(lr_u[m][r]) * lr_v[n][r] before the bias, with
    // lr_u fp32 (M x lr_rank, row stride lr_ldu, 16-byte aligned rows) and
    // lr_v fp16 bits (N x lr_rank, row stride lr_ldv, 16-byte aligned rows)
    const float *lr_u = nullptr;
    const uint16_t *lr_v = nullptr;
    int64_t lr_ldu = 0, lr_ldv = 0;
    int lr_rank = 0;
};

// Tile configurations of the square/rectangular tile kernel. The index is
// stable (it names the configuration in profiles and the ablation override).
enum TileCfg {
    CFG_256x256 = 0,        // 4 waves of 128x128, BK = 64 bytes of K, 4-stage LDS ring
    CFG_128x128 = 1,        // 4 waves of 64x64,   BK = 64 B,  4 stages
    CFG_64x64 = 2,          // 4 waves of 32x32,   BK = 128 B, 3 stages
    CFG_256x128 = 3,        // 4 waves of 128x64,  BK = 128 B, 3 stages
    CFG_256x256_BK128 = 4,  // 4 waves of 128x128, BK = 128 B, 2 stages
    CFG_128x256 = 5,        // 4 waves of 64x128,  BK = 128 B, 3 stages
    CFG_128x128_BK128 = 6,  // 4 waves of 64x64,   BK = 128 B, 4 stages
    CFG_256x256_W8 = 7,     // 8 waves of 64x128,  BK = 128 B, 2 stages
    CFG_256x256_W8_BK64 = 8,// 8 waves of 64x128,  BK = 64 B,  4 stages
    CFG_256x128_2B = 9,     // 4 waves of 128x64, BK = 64 B, 3 stages: 72 KiB, two blocks per CU
    CFG_128x128_2B = 10,    // 4 waves of 64x64, BK = 128 B, 2 stages: 64 KiB, two blocks per CU
    CFG_128x256_2B = 11,    // 4 waves of 64x128, BK = 64 B, 3 stages: 72 KiB, two blocks per CU
    CFG_256x256_PP = 12,    // 8 waves of 128x64 in two ping-pong groups, BK = 128 B, 2 stages
    // one-change ablations of CFG_256x256_BK128 (the ring kernel's VAR parameter)
    CFG_256x256_SPLIT = 13, // separate loader wavefronts for A and for B
    CFG_256x256_NT = 14,    // tile loads non-temporal (nt)
    CFG_256x256_SC1 = 15,   // tile loads at device scope (sc1)
    CFG_256x256_VGPR = 16,  // tile loads staged through VGPRs instead of direct-to-LDS
    CFG_256x256_SPREAD = 17,// the next stage's loads issued a few per k-step instead of all at once
    CFG_256x256_DTV = 18,   // B straight from global memory into MFMA registers, only A through LDS
    CFG_256x256_SC0 = 19,   // (ablation of CFG_256x256_BK128) tile loads with the sc0 cache-policy bit
    CFG_256x256_EARLY = 20, // (ablation of CFG_256x256_BK128) fragment reads fenced ahead of each k-step's MFMAs
    CFG_256x256_WEAVE = 21, // (ablation of CFG_256x256_BK128) fragment reads woven between a k-step's first MFMAs
    CFG_64x64_DEEP = 22,    // 4 waves of 32x32, BK = 128 B, 8 stages: a short K loop wholly in flight
    CFG_COUNT
};

const char *tile_cfg_name(int cfg);
int choose_tile_cfg(int prec, int64_t M, int64_t N, int64_t kbytes, int cu_count);

// Device memory of a handle that stream-K launches use: partial tiles and one
// arrival counter per split tile (all counters zero between launches).
struct TileWorkspace {
    void *partial;
    int64_t partial_bytes;
    int *flags;
    int flag_count;
};

// Arguments of the stream-K kernel: tiles [0, tiles_dp) run whole,
// round-robin over the grid; the K iterations of the other tiles (iters in
// total) are split evenly over the grid. partial holds 2 tiles of BM x BN
// 4-byte accumulators per workgroup.
struct StreamKArgs {
    int tiles_dp;
    int64_t iters;
    void *partial;
    int partial_bytes;
    int *flags;
};

// grid == 0: data-parallel launch (one workgroup per tile).
struct StreamKPlan {
    int grid;
    int tiles_dp;
    int sk_tiles;
    int64_t iters;
};

// Stream-K policy: MODE_AUTO decides by the fill of the last wave of tiles,
// MODE_OFF never splits, MODE_ON splits whenever the tiles do not fill whole
// waves of the grid (the ablation override).
// SK_MODE_PERSIST: the stream-K kernel with every tile whole (a persistent
// data-parallel grid of the resident workgroups; a measured alternative)
enum StreamKMode { SK_MODE_AUTO = -1, SK_MODE_OFF = 0, SK_MODE_ON = 1, SK_MODE_PERSIST = 2 };
StreamKPlan plan_stream_k(int cfg, int64_t M, int64_t N, int64_t kbytes, int cu_count,
                          int64_t partial_bytes, int flag_count, int mode);
// Transposed-B control: B (the B^T of the K x N layout) rows are k, ldb_b
// their byte stride; 16-byte aligned operands; PREC_F16, PREC_I8, PREC_I4.
hipError_t launch_gemm_kn(int prec, const GemmProblem &p, hipStream_t stream);
hipError_t launch_gemm(int prec, int cfg, const GemmProblem &p, const StreamKPlan &sk,
                       const TileWorkspace &ws, hipStream_t stream);

// Weight-only INT4 GEMM Y = X * dequant(Wq)^T.
struct W4A16Problem {
    const uint16_t *X;   // M x K fp16
    const uint8_t *W;    // N x K packed int4
    const uint16_t *S;   // N x K/G fp16 scales
    uint16_t *Y;         // M x N fp16
    int64_t ldx, ldw_b, lds, ldy;
    int M, N, K, G;
};

// Kernel configurations of the weight-only path (index stable, as for TileCfg).
enum W4A16Cfg {
    W4A16_MFMA_DECODE = 0,  // 16x16x32 MFMA, 16 weight rows per workgroup, K split over 4 wavefronts
    W4A16_MFMA_TILE = 1,    // 16x16x32 MFMA, 32 x 64 output tiles
    W4A16_GEMV_R1_KS2 = 2,  // VALU GEMV, 1 weight row per wavefront, K split over 2 wavefronts
    W4A16_GEMV_R2_KS2 = 3,
    W4A16_GEMV_R4_KS2 = 4,
    W4A16_GEMV_R2_KS1 = 5,  // ... whole K per wavefront
    W4A16_GEMV_R4_KS1 = 6,
    W4A16_GEMV_R8_KS1 = 7,
    W4A16_SLICE_16x16_K4 = 8,  // MFMA, activations resident in LDS, 16 x 16 tile, K over 4 wavefronts
    W4A16_SLICE_32x32_K2 = 9,  // ... 32 x 32 tile, 2 column x 2 K wavefronts
    W4A16_SLICE_64x128 = 10,   // ... 64 x 128 tile
    W4A16_SLICE_128x128 = 11,  // ... 128 x 128 tile
    W4A16_RING3_128x64 = 12,   // MFMA, 128 x 64 tile, activations and weights through a 3-stage LDS ring
    W4A16_RING4_128x64 = 13,   // ... 4-stage ring
    W4A16_SLICE_64x128_S4 = 14, // slice 64 x 128 over 4 stages of K (64 KiB LDS: two workgroups per CU)
    W4A16_SLICE_128x64_RING = 15, // slice 128 x 64 over 8 stages of K, activations through a 3-slot LDS ring
    W4A16_GEMV_MFMA_NW4 = 16,  // decode on MFMA: 16 weight rows per workgroup, K over 4 wavefronts (G % 128 == 0)
    W4A16_GEMV_MFMA_NW8 = 17,  // ... K over 8 wavefronts
    W4A16_PC_64x128 = 18,      // slice 64 x 128: 4 producer + 4 consumer wavefronts around a 4-slot LDS ring
    W4A16_PC_64x128_C8 = 19,   // ... 4 producer + 8 consumer wavefronts (64 x 16 each)
    W4A16_GEMV_MFMA_NW16 = 20, // decode on MFMA (as 16), K over 16 wavefronts of 2 steps each
    W4A16_CFG_COUNT
};

// Split-K workspace owned by a handle: the fp32 K slices of Y.
struct W4A16Workspace {
    float *partial;
    int64_t partial_floats;
};

struct W4A16Split {
    float *partial;
    int ks, kslice, mblocks, ngroups;
};

const char *w4a16_cfg_name(int cfg);
int choose_w4a16_cfg(int64_t M, int64_t N, int64_t K);

// What a weight-only call runs, decided on the host from the sizes alone:
// the configuration after fallbacks and, for the slice kernels, the split of
// K over workgroups (ks slices of kslice k; ks = 1: no second kernel).
struct W4A16Plan {
    int cfg;
    int ks;
    int kslice;
    int mblocks, ngroups;
};
W4A16Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int cfg, int cu_count, int64_t partial_floats);
hipError_t launch_w4a16(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                        hipStream_t stream);

// Argument checks of a weight-only call (all but the handle; *noop set for
// M == 0 or N == 0) and the problem they describe; shared by the handle and
// the allocation-free entry points. w4a16_split_floats: the fp32 slice
// capacity a handle gives the K split (the plan both entry points use).
mpgemm_status_t check_w4a16_args(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                                 const uint8_t *Wq, int64_t ldw, const uint16_t *S, int64_t lds,
                                 int64_t group_size, const uint16_t *Y, int64_t ldy, bool *noop);
W4A16Problem make_w4a16_problem(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                                const uint8_t *Wq, int64_t ldw, const uint16_t *S, int64_t lds,
                                int64_t group_size, uint16_t *Y, int64_t ldy);
int64_t w4a16_split_floats();
// Bytes of fp32 K slices a plan writes (0: no split).
int64_t w4a16_plan_scratch_floats(const W4A16Plan &plan);

// Symmetric INT4 quantisation of fp16 weights per (row, G-wide K group).
struct QuantizeW4Problem {
    const uint16_t *W;   // N x K fp16
    uint8_t *Q;          // N x K packed int4
    uint16_t *S;         // N x K/G fp16 scales
    int64_t ldw, ldq_b, lds;
    int N, K, G;
};

hipError_t launch_quantize_w4(const QuantizeW4Problem &p, hipStream_t stream);

// Down-projection of the W4A4 low-rank branch, U = X LD^T: X (M x K fp16
// bits, row stride ldx), LD (R x K, row stride ldd), U fp32 (M x R, row
// stride ldu). Needs K % 64 == 0, 1 <= R <= 64, X and LD 16-byte aligned with
// 16-byte aligned rows (the caller checks; other shapes take the tile GEMM).
struct LowRankDown {
    const uint16_t *X, *LD;
    float *U;
    int64_t ldx, ldd, ldu;
    int M, K, R;
};
hipError_t launch_lowrank_down(const LowRankDown &p, hipStream_t stream);

}  // namespace mpg
