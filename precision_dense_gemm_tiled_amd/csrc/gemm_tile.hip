// Tiled MFMA GEMM C = A * B^T for FP16, INT8 and packed INT4 on gfx950.
//
// Method ("Hand-Written PTX Tensor-Core GEMM Kernels: A Multi-Precision Study
// on NVIDIA L4", summary and abstract): one output tile per workgroup split
// into per-wavefront sub-tiles, the same tiling for every precision; a
// double-buffered pipeline that fetches the next K tile while the current one
// is multiplied; fragment loads from shared memory feeding the matrix unit.
// On gfx950 that becomes: coalesced 16-byte global loads of the next K tile
// into registers, an XOR-swizzled two-stage LDS ring, ds_read_b128 fragments,
// and v_mfma 32x32 instructions (f16 -> f32, i8 -> i32).
//
// INT4 has no matrix instruction on gfx950, so packed nibbles are widened in
// registers right before the i8 MFMA (the summary's INT4 paragraph: the
// expansion must not be a divergent software sequence). Each 32-bit word of 8
// packed nibbles becomes two words of int8 with no sign arithmetic:
//   w & 0xF0F0F0F0         = bytes 16 * q_odd   (high nibbles, already signed)
//   (w << 4) & 0xF0F0F0F0  = bytes 16 * q_even
// The MFMA then sums 256 * q_a * q_b exactly in int32 (|.| <= 2^14 * K), and
// the epilogue shifts right by 8. A and B go through the same widening, so
// the order in which k values reach the MFMA is the same on both sides and
// the dot product is unchanged.
#include "mpgemm_internal.h"

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int P> struct AccOf { typedef i32x16 type; typedef int32_t out; };
template <> struct AccOf<PREC_F16> { typedef f32x16 type; typedef float out; };

// XOR swizzle of the 16-byte chunk position within an LDS row. Fragment reads
// take one chunk column across 8 (or 16) consecutive rows; the swizzle spreads
// those rows over distinct banks whether the LDS serves 8 lanes x 16 B or
// 16 lanes x 16 B per cycle. Rows of CPR chunks of 16 bytes.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CPR == 8)
        return (row & 7) ^ ((row >> 3) & 1);
    else if constexpr (CPR == 4)
        return ((row >> 1) & 3) ^ ((row >> 3) & 1);
    else
        static_assert(CPR == 8 || CPR == 4, "unsupported LDS row width");
}

// Workgroup id -> output tile. Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs, each with its own L2; give every XCD a
// contiguous range of logical tiles, then walk the logical range in groups of
// GROUP_M tile rows so concurrently running tiles share A rows and B rows.
__device__ __forceinline__ void tile_of_block(int bid, int nblk, int tiles_m, int tiles_n,
                                              int &tm, int &tn) {
    constexpr int XCDS = 8, GROUP_M = 8;
    int logical = bid;
    if (nblk >= XCDS) {
        int xcd = bid % XCDS, local = bid / XCDS;
        int base = nblk / XCDS, rem = nblk % XCDS;
        logical = xcd * base + (xcd < rem ? xcd : rem) + local;
    }
    int per_group = GROUP_M * tiles_n;
    int group = logical / per_group;
    int first_m = group * GROUP_M;
    int gsize = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    int in_group = logical - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Load one 16-byte chunk of a row, zero-filling bytes at or beyond `limit`
// (the row's K extent in bytes). `off` is the chunk's byte offset in the row.
__device__ __forceinline__ i32x4 load_chunk(const uint8_t *row, int64_t off, int64_t limit,
                                            bool row_ok) {
    i32x4 v = {0, 0, 0, 0};
    if (row_ok && off < limit) {
        if (off + 16 <= limit) {
            v = *reinterpret_cast<const i32x4 *>(row + off);
        } else {
            // ragged K tail: only whole elements exist past this point, byte
            // granularity covers every precision
            uint8_t b[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                b[i] = (off + i < limit) ? row[off + i] : 0;
            v = *reinterpret_cast<const i32x4 *>(b);
        }
    }
    return v;
}

template <int P, int BM, int BN, int BKB, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tile_kernel(GemmProblem p, int tiles_m,
                                                                   int tiles_n) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int CPR = BKB / 16;
    constexpr int A_PER_T = BM * CPR / NT, B_PER_T = BN * CPR / NT;
    constexpr int STAGE = (BM + BN) * BKB;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "staging must divide evenly");
    static_assert(CPR % 2 == 0, "two lane groups read adjacent chunks");
    // LDS budget, checked at build time (160 KiB per workgroup on gfx950).
    static_assert(2 * STAGE <= 160 * 1024, "LDS ring exceeds 160 KiB");

    typedef typename AccOf<P>::type acc_t;
    typedef typename AccOf<P>::out out_t;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WGN) * WTM;
    const int wn0 = (wave % WGN) * WTN;

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;

    const int64_t kbytes = p.kbytes;
    const int KT = (int)((kbytes + BKB - 1) / BKB);

    // Per-thread staging: chunk q = i * NT + tid of the A (then B) tile.
    i32x4 stg[A_PER_T + B_PER_T];

    auto load_tile = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BKB;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            int q = i * NT + tid, r = q / CPR, c = q % CPR;
            int gr = row0 + r;
            bool ok = gr < p.M;
            const uint8_t *rowp = p.A + (int64_t)(ok ? gr : 0) * p.lda_b;
            stg[i] = load_chunk(rowp, k0 + c * 16, kbytes, ok);
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            int q = i * NT + tid, r = q / CPR, c = q % CPR;
            int gr = col0 + r;
            bool ok = gr < p.N;
            const uint8_t *rowp = p.B + (int64_t)(ok ? gr : 0) * p.ldb_b;
            stg[A_PER_T + i] = load_chunk(rowp, k0 + c * 16, kbytes, ok);
        }
    };
    auto store_tile = [&](int stage) {
        uint8_t *As = smem + stage * STAGE;
        uint8_t *Bs = As + BM * BKB;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            int q = i * NT + tid, r = q / CPR, c = q % CPR;
            *reinterpret_cast<i32x4 *>(As + r * BKB + ((c ^ swz<CPR>(r)) * 16)) = stg[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            int q = i * NT + tid, r = q / CPR, c = q % CPR;
            *reinterpret_cast<i32x4 *>(Bs + r * BKB + ((c ^ swz<CPR>(r)) * 16)) = stg[A_PER_T + i];
        }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = acc_t{};

    auto compute = [&](int stage) {
        const uint8_t *As = smem + stage * STAGE;
        const uint8_t *Bs = As + BM * BKB;
        const int g = lane >> 5;
#pragma unroll
        for (int kc = 0; kc < CPR; kc += 2) {
            const int c = kc + g;
            i32x4 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                int r = wm0 + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const i32x4 *>(As + r * BKB + ((c ^ swz<CPR>(r)) * 16));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                int r = wn0 + j * 32 + (lane & 31);
                b[j] = *reinterpret_cast<const i32x4 *>(Bs + r * BKB + ((c ^ swz<CPR>(r)) * 16));
            }
            if constexpr (P == PREC_I8) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
            } else if constexpr (P == PREC_F16) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, a[i]), __builtin_bit_cast(f16x8, b[j]),
                            acc[i][j], 0, 0, 0);
            } else {
                const int M4 = (int)0xF0F0F0F0u;
                i32x4 ah[TM], al[TM], bh[TN], bl[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    ah[i] = a[i] & M4;
                    al[i] = (a[i] << 4) & M4;
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    bh[j] = b[j] & M4;
                    bl[j] = (b[j] << 4) & M4;
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah[i], bh[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(al[i], bl[j], acc[i][j], 0, 0, 0);
                    }
            }
        }
    };

    if (KT > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load_tile(kt + 1);
        compute(cur);
        if (kt + 1 < KT)
            store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue. 32x32 accumulator layout: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
    out_t *C = reinterpret_cast<out_t *>(p.C);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = col0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < p.M && col < p.N) {
                    if constexpr (P == PREC_I4)
                        C[(int64_t)row * p.ldc + col] = acc[i][j][r] >> 8;
                    else
                        C[(int64_t)row * p.ldc + col] = acc[i][j][r];
                }
            }
        }
}

// ------------------------------------------------------------------ launch

struct CfgShape { int BM, BN; const char *name; };
static const CfgShape kCfg[CFG_COUNT] = {
    {256, 256, "256x256x64B_w2x2"},
    {128, 128, "128x128x64B_w2x2"},
    {64, 64, "64x64x128B_w2x2"},
    {256, 128, "256x128x64B_w2x2"},
};

const char *tile_cfg_name(int cfg) {
    return (cfg >= 0 && cfg < CFG_COUNT) ? kCfg[cfg].name : "invalid";
}

int choose_tile_cfg(int prec, int64_t M, int64_t N, int64_t kbytes, int cu_count) {
    (void)prec;
    (void)kbytes;
    auto tiles = [&](int c) {
        return ((M + kCfg[c].BM - 1) / kCfg[c].BM) * ((N + kCfg[c].BN - 1) / kCfg[c].BN);
    };
    // Largest tile that still gives every compute unit a workgroup.
    if (tiles(CFG_256x256) >= cu_count)
        return CFG_256x256;
    if (tiles(CFG_256x128) >= cu_count)
        return CFG_256x128;
    if (tiles(CFG_128x128) >= cu_count / 2)
        return CFG_128x128;
    return CFG_64x64;
}

template <int P, int BM, int BN, int BKB, int WGM, int WGN>
static hipError_t launch_one(const GemmProblem &p, hipStream_t stream) {
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    dim3 grid(tiles_m * tiles_n), block(64 * WGM * WGN);
    hipLaunchKernelGGL((gemm_tile_kernel<P, BM, BN, BKB, WGM, WGN>), grid, block, 0, stream, p,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_prec(int cfg, const GemmProblem &p, hipStream_t stream) {
    switch (cfg) {
    case CFG_256x256: return launch_one<P, 256, 256, 64, 2, 2>(p, stream);
    case CFG_128x128: return launch_one<P, 128, 128, 64, 2, 2>(p, stream);
    case CFG_64x64: return launch_one<P, 64, 64, 128, 2, 2>(p, stream);
    case CFG_256x128: return launch_one<P, 256, 128, 64, 2, 2>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(int prec, int cfg, const GemmProblem &p, hipStream_t stream) {
    switch (prec) {
    case PREC_F16: return launch_prec<PREC_F16>(cfg, p, stream);
    case PREC_I8: return launch_prec<PREC_I8>(cfg, p, stream);
    case PREC_I4: return launch_prec<PREC_I4>(cfg, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mpg
