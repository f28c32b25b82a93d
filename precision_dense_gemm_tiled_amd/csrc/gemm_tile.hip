// Tiled MFMA GEMM C = A * B^T for FP16, INT8 and packed INT4 on gfx950.
//
// Method ("Hand-Written PTX Tensor-Core GEMM Kernels: A Multi-Precision Study
// on NVIDIA L4", summary and abstract): one output tile per workgroup split
// into per-wavefront sub-tiles, the same tiling for every precision; a
// double-buffered pipeline that fetches the next K tile while the current one
// is multiplied; fragment loads from shared memory feeding the matrix unit.
// On gfx950 that becomes: coalesced 16-byte direct-to-LDS loads
// (global_load_lds_dwordx4) of the next K tile into an XOR-swizzled two-stage
// LDS ring, ds_read_b128 fragments double-buffered in registers, and v_mfma
// 32x32 instructions (f16 -> f32, i8 -> i32), with the memory instructions
// issued in the shadow of the MFMAs.
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
#include "lds_dma.h"

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int P> struct AccOf { typedef i32x16 type; typedef int32_t out; typedef int elem; };
template <> struct AccOf<PREC_F16> { typedef f32x16 type; typedef float out; typedef float elem; };
template <> struct AccOf<PREC_W4A4> { typedef i32x16 type; typedef uint16_t out; typedef int elem; };

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

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2: renumber them so every XCD holds a contiguous range of
// logical ids.
__device__ __forceinline__ int xcd_logical(int bid, int nblk) {
    constexpr int XCDS = 8;
    if (nblk < XCDS)
        return bid;
    const int xcd = bid % XCDS, local = bid / XCDS;
    const int base = nblk / XCDS, rem = nblk % XCDS;
    return xcd * base + (xcd < rem ? xcd : rem) + local;
}

// Logical tile index -> output tile: walk the tiles in groups of GROUP_M tile
// rows so concurrently running tiles share A rows and B rows in L2.
__device__ __forceinline__ void tile_raster(int logical, int tiles_m, int tiles_n, int &tm, int &tn) {
    constexpr int GROUP_M = 8;
    const int per_group = GROUP_M * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * GROUP_M;
    const int gsize = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Workgroup id -> output tile when the grid has one workgroup per tile.
__device__ __forceinline__ void tile_of_block(int bid, int nblk, int tiles_m, int tiles_n,
                                              int &tm, int &tn) {
    tile_raster(xcd_logical(bid, nblk), tiles_m, tiles_n, tm, tn);
}

// Zero the bytes of a 16-byte chunk at positions >= nvalid (0 <= nvalid <= 16).
__device__ __forceinline__ i32x4 keep_bytes(i32x4 v, int nvalid) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        int nb = nvalid - 4 * d;
        uint32_t m = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u));
        v[d] &= (int)m;
    }
    return v;
}

// Chunk load with K masking for 16-byte aligned rows. A chunk whose first
// byte lies in the row is read whole: it is 16-byte aligned, so it cannot
// cross a page boundary, and the bytes past the row's K extent are cleared in
// registers.
__device__ __forceinline__ i32x4 load_chunk_masked(const uint8_t *row, int64_t off, int64_t limit,
                                                   bool row_ok) {
    i32x4 v = {0, 0, 0, 0};
    if (row_ok && off < limit) {
        v = *reinterpret_cast<const i32x4 *>(row + off);
        if (off + 16 > limit)
            v = keep_bytes(v, (int)(limit - off));
    }
    return v;
}

// Chunk load for rows with no alignment guarantee: byte gathers.
__device__ __forceinline__ i32x4 load_chunk_bytes(const uint8_t *row, int64_t off, int64_t limit,
                                                  bool row_ok) {
    uint32_t w[4] = {0, 0, 0, 0};
    if (row_ok) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (off + i < limit)
                w[i >> 2] |= (uint32_t)row[off + i] << (8 * (i & 3));
    }
    return i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

// MFMAs of one k-step (32 bytes of K per row: one chunk per lane group) on
// fragments already in registers, restricted to the blocks (i, j) whose flat
// index i * TN + j lies in [LO, HI). With TRANS the two operands trade
// places, so each accumulator block holds the transpose of its C block
// (store_tile_lds reads that layout).
template <int P, int TM, int TN, int LO = 0, int HI = TM * TN, bool TRANS = false>
__device__ __forceinline__ void mfma_step(const i32x4 (&a)[TM], const i32x4 (&b)[TN],
                                          typename AccOf<P>::type (&acc)[TM][TN]) {
#pragma unroll
    for (int f = LO; f < HI; ++f) {
        const int i = f / TN, j = f % TN;
        const i32x4 x = TRANS ? b[j] : a[i];
        const i32x4 y = TRANS ? a[i] : b[j];
        if constexpr (P == PREC_I8) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x, y, acc[i][j], 0, 0, 0);
        } else if constexpr (P == PREC_F16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), acc[i][j], 0, 0, 0);
        } else {
            // INT4: widen both operands (16 * nibble per byte) right before use
            const int M4 = (int)0xF0F0F0F0u;
            const i32x4 xh = x & M4, xl = (x << 4) & M4;
            const i32x4 yh = y & M4, yl = (y << 4) & M4;
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xh, yh, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xl, yl, acc[i][j], 0, 0, 0);
        }
    }
}

// ds_read_b128 fragments of one k-step (32 bytes of K per row, one 16-byte
// chunk per lane group) of an LDS stage.
template <int BM, int BKB, int TM, int TN>
__device__ __forceinline__ void read_frags(const uint8_t *As, int step, int wm0, int wn0, int lane,
                                           i32x4 (&a)[TM], i32x4 (&b)[TN]) {
    constexpr int CPR = BKB / 16;
    const uint8_t *Bs = As + BM * BKB;
    const int c = 2 * step + (lane >> 5);
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
}

// The W4A4 low-rank term of one row of 32 x 32 output blocks (rows row_b ...
// row_b + 31, columns col0 + 32 j + lane % 32 for the TN blocks j): sum over
// r of fp16(U[m][r]) * V[n][r] ("Warp-Specialized Kernel Implementation for
// W4A4 MatMul on Latest GPU Architectures", section 1: the low-rank residual
// L(X) next to the 4-bit product), on the matrix unit in the accumulator
// layout of the blocks, 16 of rank per v_mfma_f32_32x32x16_f16. Lane l
// supplies row row_b + l % 32 of U (its fp32 values rounded to fp16, nearest
// even, once per row of blocks) and column l % 32 of each block's V rows,
// ranks 8 (l / 32) ... + 7 of each 16. Rows and columns past the problem are
// clamped (their outputs are not stored).
template <int TN, bool TRANS = false>
__device__ __forceinline__ void lowrank_row(const GemmProblem &p, int row_b, int col0, f32x16 (&lr)[TN]) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int m = min(row_b + (lane & 31), p.M - 1);
    const float *u = p.lr_u + (int64_t)m * p.lr_ldu + 8 * (lane >> 5);
    const uint16_t *v[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = min(col0 + 32 * j + (lane & 31), p.N - 1);
        v[j] = p.lr_v + (int64_t)n * p.lr_ldv + 8 * (lane >> 5);
    }
    auto to_f16 = [](f32x4 x0, f32x4 x1) {
        return f16x8{(_Float16)x0[0], (_Float16)x0[1], (_Float16)x0[2], (_Float16)x0[3],
                     (_Float16)x1[0], (_Float16)x1[1], (_Float16)x1[2], (_Float16)x1[3]};
    };
    // 32 ranks per pass (the rank is a multiple of 16: the last pass may hold
    // one step only, and then reads nothing past it)
    for (int t = 0; t < p.lr_rank; t += 32) {
        const bool two = t + 16 < p.lr_rank;
        const f16x8 a0 = to_f16(*reinterpret_cast<const f32x4 *>(u + t), *reinterpret_cast<const f32x4 *>(u + t + 4));
        f16x8 a1 = {};
        f16x8 b0[TN], b1[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b0[j] = *reinterpret_cast<const f16x8 *>(v[j] + t);
        if (two) {
            a1 = to_f16(*reinterpret_cast<const f32x4 *>(u + t + 16), *reinterpret_cast<const f32x4 *>(u + t + 20));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b1[j] = *reinterpret_cast<const f16x8 *>(v[j] + t + 16);
        }
        // TRANS: operands swapped, so each block holds its transpose (the
        // layout of the main loop's transposed accumulators)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            lr[j] = TRANS ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b0[j], a0, lr[j], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0[j], lr[j], 0, 0, 0);
        if (two) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                lr[j] = TRANS ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b1[j], a1, lr[j], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1[j], lr[j], 0, 0, 0);
        }
    }
}

// Epilogue. 32x32 accumulator layout: register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
template <int P, int TM, int TN>
__device__ __forceinline__ void store_tile(const GemmProblem &p, int row0, int col0, int lane,
                                           const typename AccOf<P>::type (&acc)[TM][TN],
                                           const float *fx = nullptr, const float *fw = nullptr,
                                           const float *fb = nullptr) {
    typedef typename AccOf<P>::out out_t;
    out_t *C = reinterpret_cast<out_t *>(p.C);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // the W4A4 low-rank term of this row of blocks (zero without one)
        [[maybe_unused]] f32x16 lr[TN];
        if constexpr (P == PREC_W4A4) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                lr[j] = f32x16{};
            if (p.lr_rank > 0)
                lowrank_row<TN>(p, row0 + i * 32, col0, lr);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int cl = j * 32 + (lane & 31);   // column within this wavefront's sub-tile
            const int col = col0 + cl;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int row = row0 + rl;
                if (row < p.M && col < p.N) {
                    if constexpr (P == PREC_W4A4) {
                        // |acc >> 8| <= 64 K < 2^24: exact in fp32; then two
                        // products, the low-rank term (0 without one) and the
                        // bias in fp32, each rounded on its own (no fused
                        // multiply-add), one rounding to fp16
#pragma clang fp contract(off)
                        const float y = ((float)(acc[i][j][r] >> 8) * fx[rl] * fw[cl] + lr[j][r]) + fb[cl];
                        C[(int64_t)row * p.ldc + col] = __builtin_bit_cast(uint16_t, (_Float16)y);
                    } else if constexpr (P == PREC_I4) {
                        C[(int64_t)row * p.ldc + col] = acc[i][j][r] >> 8;
                    } else {
                        C[(int64_t)row * p.ldc + col] = acc[i][j][r];
                    }
                }
            }
        }
    }
}

// Epilogue for transposed accumulators (mfma_step with TRANS): register r
// of lane l in block (i, j) holds row 32 i + l % 32 and column
// 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 of the wavefront's WTM x WTN
// sub-tile, so each group of four registers is four consecutive columns of
// one row. The wavefront stages RP rows at a time in its own LDS region
// (row-major, WTN * 4 bytes per row, 16-byte chunk c of row r stored at
// chunk c ^ (r & 15), which keeps both the writes and the read-back free of
// bank conflicts), then reads whole row segments back and writes C with
// 16-byte stores (per-element stores at the right and bottom edges, or when
// C rows are not 16-byte aligned). Only this wavefront touches its region:
// no barrier between the passes.
template <int P, int TM, int TN, int RP>
__device__ __forceinline__ void store_tile_lds(const GemmProblem &p, uint8_t *region, int row0, int col0,
                                               int lane, const typename AccOf<P>::type (&acc)[TM][TN]) {
    typedef typename AccOf<P>::out out_t;
    typedef out_t out4 __attribute__((ext_vector_type(4)));
    constexpr int WTN = TN * 32, RB = WTN * 4, CPW = WTN / 4;   // bytes and 16-byte chunks per row
    static_assert(CPW >= 16 && RP % 32 == 0 && (TM * 32) % RP == 0 && (RP * CPW) % 64 == 0, "staging shape");
    out_t *C = reinterpret_cast<out_t *>(p.C);
    const bool vec = p.c_vec16 != 0;
#pragma unroll
    for (int pass = 0; pass < TM * 32 / RP; ++pass) {
#pragma unroll
        for (int ib = 0; ib < RP / 32; ++ib) {
            const int i = pass * (RP / 32) + ib;
            const int rl = ib * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = 8 * j + 2 * g + (lane >> 5);
                    out4 v;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        if constexpr (P == PREC_I4)
                            v[d] = acc[i][j][4 * g + d] >> 8;
                        else
                            v[d] = acc[i][j][4 * g + d];
                    }
                    *reinterpret_cast<out4 *>(region + rl * RB + ((c ^ (rl & 15)) * 16)) = v;
                }
        }
#pragma unroll
        for (int q = 0; q < RP * CPW / 64; ++q) {
            const int f = q * 64 + lane;
            const int rl = f / CPW, c = f % CPW;
            const out4 v = *reinterpret_cast<const out4 *>(region + rl * RB + ((c ^ (rl & 15)) * 16));
            const int row = row0 + pass * RP + rl, col = col0 + c * 4;
            if (row < p.M) {
                out_t *dst = C + (int64_t)row * p.ldc + col;
                if (vec && col + 3 < p.N) {
                    // non-temporal: C is written once and never read back
                    // here, so it should not displace A and B lines that
                    // later tiles still read from the caches
                    __builtin_nontemporal_store(v, reinterpret_cast<out4 *>(dst));
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        if (col + d < p.N)
                            dst[d] = v[d];
                }
            }
        }
    }
}

// W4A4 epilogue for transposed accumulators (the layout store_tile_lds
// reads: register r of lane l in block (i, j) holds row 32 i + l % 32 and
// column 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 of the wavefront's sub-tile).
// Each output is computed in registers exactly as in store_tile:
// fp16((((acc >> 8) * sx) * sw + low-rank term) + bias), each fp32 operation
// rounded on its own; four consecutive columns are packed into 8 bytes and
// staged RP rows at a time in the wavefront's own LDS region (row-major fp16,
// 16-byte chunk c of row r at chunk c ^ (r % CPW)), then whole row segments
// are read back and written with 16-byte stores (per-element stores at the
// right edge, or when C rows are not 16-byte aligned). fx / fw / fb: the
// staged row factors, column factors and bias of this sub-tile.
template <int TM, int TN, int RP>
__device__ __forceinline__ void store_tile_lds_w4a4(const GemmProblem &p, uint8_t *region, int row0, int col0,
                                                    int lane, const i32x16 (&acc)[TM][TN], const float *fx,
                                                    const float *fw, const float *fb) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int WTN = TN * 32, RB = WTN * 2, CPW = WTN / 8;   // bytes and 16-byte chunks per staged row
    static_assert((CPW == 8 || CPW == 16) && RP % 32 == 0 && (TM * 32) % RP == 0 && (RP * CPW) % 64 == 0,
                  "staging shape");
    uint16_t *C = reinterpret_cast<uint16_t *>(p.C);
    const bool vec = p.c_vec16 != 0 && p.ldc % 8 == 0;
    const int h = lane >> 5;
#pragma unroll
    for (int pass = 0; pass < TM * 32 / RP; ++pass) {
#pragma unroll
        for (int ib = 0; ib < RP / 32; ++ib) {
            const int i = pass * (RP / 32) + ib;
            const int rl = ib * 32 + (lane & 31);
            const float sx = fx[i * 32 + (lane & 31)];
            f32x16 lr[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                lr[j] = f32x16{};
            if (p.lr_rank > 0)
                lowrank_row<TN, true>(p, row0 + i * 32, col0, lr);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int cl = 32 * j + 8 * g + 4 * h;
                    const f32x4 wv = *reinterpret_cast<const f32x4 *>(fw + cl);
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(fb + cl);
                    u16x4 v;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma clang fp contract(off)
                        const float y = ((float)(acc[i][j][4 * g + d] >> 8) * sx * wv[d] + lr[j][4 * g + d]) + bv[d];
                        v[d] = __builtin_bit_cast(uint16_t, (_Float16)y);
                    }
                    const int c = 4 * j + g;
                    *reinterpret_cast<u16x4 *>(region + rl * RB + ((c ^ (rl & (CPW - 1))) * 16) + 8 * h) = v;
                }
        }
#pragma unroll
        for (int q = 0; q < RP * CPW / 64; ++q) {
            const int f = q * 64 + lane;
            const int rl = f / CPW, c = f % CPW;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(region + rl * RB + ((c ^ (rl & (CPW - 1))) * 16));
            const int row = row0 + pass * RP + rl, col = col0 + c * 8;
            if (row < p.M) {
                uint16_t *dst = C + (int64_t)row * p.ldc + col;
                if (vec && col + 7 < p.N) {
                    // non-temporal: Y is written once and never read back here
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                } else {
#pragma unroll
                    for (int d = 0; d < 8; ++d)
                        if (col + d < p.N)
                            dst[d] = (uint16_t)(v[d / 2] >> (16 * (d % 2)));
                }
            }
        }
    }
}

// W4A4 epilogue factors of a BM x BN tile staged in LDS as fp32 (the operand
// buffers are free once every wavefront is past its last fragment read):
// fac[0, BM) = SX of the tile's rows, fac[BM, BM + BN) = SW of its columns,
// fac[BM + BN, BM + 2 BN) = bias (0 without one). Entries past M or N are 0.
template <int BM, int BN, int NT>
__device__ __forceinline__ void stage_factors(const GemmProblem &p, int row0, int col0, int tid,
                                              float *fac) {
    __syncthreads();
    for (int t = tid; t < BM; t += NT)
        fac[t] = row0 + t < p.M ? (float)__builtin_bit_cast(_Float16, p.sx[row0 + t]) : 0.f;
    for (int t = tid; t < BN; t += NT) {
        const bool ok = col0 + t < p.N;
        fac[BM + t] = ok ? (float)__builtin_bit_cast(_Float16, p.sw[col0 + t]) : 0.f;
        fac[BM + BN + t] = ok && p.bias ? (float)__builtin_bit_cast(_Float16, p.bias[col0 + t]) : 0.f;
    }
    __syncthreads();
}

// Main loop for 16-byte aligned operands whose BM (BN) rows span less than
// 2^31 bytes: accumulates pipeline entries [e0, e1) of output tile
// (row0, col0) into acc. Full K tiles move from global memory straight into
// an NS-stage LDS ring with direct-to-LDS loads (no staging registers, no
// ds_write), NS - 1 tiles ahead of the MFMAs that consume them. One load
// instruction of a wavefront fills 1 KiB of contiguous LDS, i.e. 64 / CPR
// whole rows of a tile; lane l lands at row l / CPR, 16-byte slot l % CPR, so
// it fetches the global chunk that the XOR swizzle puts in that slot. Each
// thread's rows are r0 + i * RS (RS = NT / CPR), whose swizzle is the same for
// every i, so its addresses are one uniform block base plus one 32-bit offset
// per load.
//
// Entries: if K is not a multiple of BKB, entry 0 is the partial K tile
// (loaded through registers with K masking); entry e >= NPRE is full K tile
// e - NPRE. The caller guarantees 0 <= e0 < e1 <= KT and that the ring is
// free (no wavefront still reads it). On return every load has landed.
//
// VAR selects one change at a time for the ablation configurations (the L4
// study's pipeline ablations: separate loaders for the two operands, the
// load cache policy, and on gfx950 also the staging path): 0 the kernel as
// described; 1 split loaders (the first half of the wavefronts loads every
// A row of the stage, the second half every B row); 2 the tile loads marked
// non-temporal (nt); 3 the tile loads at device scope (sc1); 4 tile loads
// staged through VGPRs (global_load_dwordx4, then ds_write_b128 into the free
// stage before the barrier that publishes it) instead of direct-to-LDS;
// 5 the next entry's loads spread over the k-steps; 6 the tile loads with
// the sc0 cache-policy bit; 7 each k-step's fragment reads fenced ahead of
// the previous step's MFMAs; 8 each k-step's fragment reads woven two per
// MFMA between its first MFMAs (and step 0's direct-to-LDS loads two per MFMA
// after them).
enum { VAR_BASE = 0, VAR_SPLIT = 1, VAR_NT = 2, VAR_SC1 = 3, VAR_VGPR = 4, VAR_SPREAD = 5, VAR_SC0 = 6,
       VAR_EARLY = 7, VAR_WEAVE = 8 };

template <int AUX>
__device__ __forceinline__ void dma16_cp(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, AUX);
}

template <int P, int BM, int BN, int BKB, int WGM, int WGN, int NS, int VAR = VAR_BASE>
struct RingTile {
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int CPR = BKB / 16;
    static constexpr int RS = NT / CPR;
    static constexpr int A_PER_T = BM / RS, B_PER_T = BN / RS;
    static constexpr int NL = A_PER_T + B_PER_T;   // direct-to-LDS loads per thread per tile
    static constexpr bool SPLIT = VAR == VAR_SPLIT;
    static constexpr bool VSTAGE = VAR == VAR_VGPR;
    // SPREAD: the next entry's loads are issued a few per k-step, between the
    // fragment reads and MFMAs, instead of all at the top of the iteration
    static constexpr bool SPREAD = VAR == VAR_SPREAD;
    // EARLY: each k-step's fragment reads are fenced ahead of the previous
    // step's MFMAs. Otherwise both share one scheduling region, and the
    // compiler sinks the reads towards the end of the step (it reuses the
    // registers of fragments already consumed), leaving a few MFMAs to cover
    // them. Measured on MI355X, the early order is 4-5 % slower at 4096 and
    // 8192 (INT8, FP16, INT4): the matrix unit idles while a wavefront
    // issues its reads ahead of its MFMAs.
    static constexpr bool EARLY = VAR == VAR_EARLY;
    static constexpr bool WEAVE = VAR == VAR_WEAVE;
    static constexpr int CPOL = VAR == VAR_NT ? 2 : (VAR == VAR_SC1 ? 16 : (VAR == VAR_SC0 ? 1 : 0));
    static constexpr int RSL = SPLIT ? RS / 2 : RS;   // rows per load round of one loader
    static constexpr int HW = NT / 128;                // wavefronts per operand when split
    static_assert(!SPLIT || (BM == BN && (NT / 2) % 64 == 0 && RSL % 16 == 0), "split loaders");
    static constexpr int STAGE = (BM + BN) * BKB;
    static constexpr int STEPS = CPR / 2;
    static constexpr int LDS_BYTES = NS * STAGE;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(NT % CPR == 0 && BM % RS == 0 && BN % RS == 0, "staging must divide evenly");
    static_assert(RS % 16 == 0, "swizzle must repeat every RS rows");
    static_assert(STEPS % 2 == 0, "k-steps per stage alternate two fragment buffers");
    static_assert(NS >= 2 && (NS - 2) * NL < 64, "ring depth");
    // LDS budget, checked at build time (160 KiB per workgroup on gfx950).
    static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KiB");
    typedef typename AccOf<P>::type acc_t;
    // Accumulators hold transposed blocks (operands swapped in the MFMA),
    // written back through LDS with 16-byte stores (store_tile_lds; for W4A4
    // store_tile_lds_w4a4, which stages fp16 outputs and keeps the tile's
    // factor table at the end of the ring).
    static constexpr bool TRANS = WTN >= 64;
    static constexpr int NW = WGM * WGN;
    static constexpr int FACB = P == PREC_W4A4 ? ((BM + 2 * BN) * 4 + 15) / 16 * 16 : 0;   // factor table
    static constexpr int OUTB = P == PREC_W4A4 ? 2 : 4;                                    // staged bytes per output
    static constexpr int REGION = (LDS_BYTES - FACB) / NW / 16 * 16;                      // per wavefront
    static constexpr int RP_MAX = REGION / (WTN * OUTB) / 32 * 32;   // rows one pass can stage
    static constexpr int RP = RP_MAX >= WTM ? WTM : (WTM % RP_MAX == 0 ? RP_MAX : 32);
    static_assert(!TRANS || (RP >= 32 && RP * WTN * OUTB <= REGION), "epilogue staging fits the ring");

    // WEAVE: instruction order of one scheduling region of NMF MFMAs: the
    // TM + TN fragment reads two after each of the first MFMAs, then (step 0)
    // the NL direct-to-LDS loads two after each following MFMA, then the
    // remaining MFMAs. The masks are the scheduler's instruction classes: 0x8
    // MFMA, 0x100 LDS read, 0x20 vector-memory read.
    template <bool WITH_DMA, int NMF>
    static __device__ __forceinline__ void weave_order() {
        constexpr int NR = TM + TN;
        constexpr int RG = (NR + 1) / 2;   // MFMAs that carry the reads
#pragma unroll
        for (int i = 0; i < RG; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        if constexpr (WITH_DMA) {
            constexpr int DG = (NL + 1) / 2;
            static_assert(RG + DG <= TM * TN, "loads fit between the MFMAs");
#pragma unroll
            for (int i = 0; i < DG; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - RG - DG, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - RG, 0);
        }
    }

    static __device__ __forceinline__ void mainloop(const GemmProblem &p, uint8_t *smem, int row0,
                                                    int col0, int e0, int e1, int tid, int lane,
                                                    int wave, acc_t (&acc)[TM][TN]) {
        const int wm0 = (wave / WGN) * WTM;
        const int wn0 = (wave % WGN) * WTN;
        const int64_t kbytes = p.kbytes;
        const int KF = (int)(kbytes / BKB);     // full K tiles
        const bool tail = (kbytes % BKB) != 0;  // plus one partial tile
        const int NPRE = tail ? 1 : 0;

        // Load i of this thread: operand A or B, row r0 + step. With split
        // loaders a wavefront loads one operand only (wave-uniform choice).
        const bool a_wave = !SPLIT || wave < HW;
        const int r0 = (SPLIT ? tid % (NT / 2) : tid) / CPR;
        const int cg = (tid % CPR) ^ swz<CPR>(r0);   // global chunk of this lane's slot
        auto ld_is_a = [&](int i) { return SPLIT ? a_wave : i < A_PER_T; };
        auto ld_step = [&](int i) { return SPLIT ? i * RSL : (i < A_PER_T ? i : i - A_PER_T) * RS; };
        const uint8_t *Ab = p.A + (int64_t)row0 * p.lda_b;
        const uint8_t *Bb = p.B + (int64_t)col0 * p.ldb_b;
        const int a_rows = p.M - row0, b_rows = p.N - col0;   // >= 1
        uint32_t off[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const bool isa = ld_is_a(i);
            const int rows = isa ? a_rows : b_rows;
            int r = r0 + ld_step(i);
            r = r < rows ? r : rows - 1;   // clamped rows feed outputs never stored
            off[i] = (uint32_t)r * (uint32_t)(isa ? p.lda_b : p.ldb_b) + cg * 16;
        }
        // wave-uniform LDS base of this wavefront's DMA rows within a stage
        const int wrow = (SPLIT ? wave % HW : wave) * (64 / CPR);
        auto ld_dst = [&](int i) { return (ld_is_a(i) ? 0 : BM * BKB) + (wrow + ld_step(i)) * BKB; };
        i32x4 R[VSTAGE ? NL : 1];   // staging registers of the VGPR-staged variant

        // Every call issues exactly NL loads (entries past the last full tile
        // re-read it into a stage that is free), so a fixed vmcnt tells which
        // entry has landed. The host sends problems with no full K tile
        // (KF == 0) to the generic kernel.
        auto dma_one = [&](int e, int i) {   // load i of entry e
            int kt = e - NPRE;
            kt = kt < KF - 1 ? kt : KF - 1;
            const uint8_t *src = (ld_is_a(i) ? Ab : Bb) + (int64_t)kt * BKB + off[i];
            if constexpr (VSTAGE)
                R[i] = *reinterpret_cast<const i32x4 *>(src);
            else
                dma16_cp<CPOL>(src, smem + (e % NS) * STAGE + ld_dst(i));
        };
        auto dma_entry = [&](int e) {
#pragma unroll
            for (int i = 0; i < NL; ++i)
                dma_one(e, i);
        };
        // the loads of entry e that go with k-step `step` (SPREAD)
        auto dma_step = [&](int e, int step) {
#pragma unroll
            for (int i = 0; i < NL; ++i)
                if (i * STEPS / NL == step)
                    dma_one(e, i);
        };
        // VGPR-staged variant: the registers of entry e -> its stage
        auto stage_regs = [&](int e) {
            if constexpr (VSTAGE) {
                uint8_t *S = smem + (e % NS) * STAGE + lane * 16;
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    *reinterpret_cast<i32x4 *>(S + ld_dst(i)) = R[i];
            }
        };
        // partial tile kt -> stage 0 through registers, bytes past K cleared
        auto reg_tail = [&](int kt) {
            const int64_t k0 = (int64_t)kt * BKB + cg * 16;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const bool isa = ld_is_a(i);
                const i32x4 v = load_chunk_masked((isa ? Ab : Bb) + (off[i] - cg * 16), k0, kbytes,
                                                  r0 + ld_step(i) < (isa ? a_rows : b_rows));
                *reinterpret_cast<i32x4 *>(smem + ld_dst(i) + lane * 16) = v;
            }
        };

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = acc_t{};

        // Prologue: entries e0 .. e0 + NS - 2 in flight; wait for entry e0 only.
        i32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
        if (tail && e0 == 0)
            reg_tail(KF);
        else {
            dma_entry(e0);
            stage_regs(e0);
        }
#pragma unroll
        for (int e = 1; e < NS - 1; ++e) {
            dma_entry(e0 + e);
            stage_regs(e0 + e);
        }
        // entry e0 has landed (through LDS DMA, or through registers: lgkmcnt)
        wait_vm_lds<(NS - 2) * NL>();
        lds_barrier();
        read_frags<BM, BKB, TM, TN>(smem + (e0 % NS) * STAGE, 0, wm0, wn0, lane, fa0, fb0);

        // One pipeline entry e in LDS stage e % NS. Region A (before the
        // barrier): the direct-to-LDS loads of entry e + NS - 1 into the stage
        // freed by entry e - 1; per k-step, the fragment reads of the next step
        // and the MFMAs of this one; the first KA MFMAs of the last step. The
        // barrier publishes entry e + 1 (its loads, issued NS - 2 entries
        // earlier, are the oldest ones outstanding) and certifies that every
        // wavefront has finished reading stage e % NS. Region B: step-0
        // fragment reads of the next stage interleaved with the rest of the
        // last step's MFMAs.
        constexpr int NMF = TM * TN;
        constexpr int KA = NMF >= 4 ? NMF / 4 : 1;
        for (int e = e0; e < e1; ++e) {
            const uint8_t *S = smem + (e % NS) * STAGE;
            const uint8_t *Snext = smem + ((e + 1) % NS) * STAGE;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!SPREAD && !EARLY && !WEAVE)
                dma_entry(e + NS - 1);
#pragma unroll
            for (int step = 0; step < STEPS - 1; ++step) {
                // one scheduling region per k-step: fragment reads of the next
                // step and the MFMAs of this one (no back-to-back MFMAs on one
                // accumulator across steps); EARLY fences the reads first
                if constexpr (SPREAD)
                    dma_step(e + NS - 1, step);
                // Only this step's fragments (read a whole step ago) can still
                // be in flight: wait for them before issuing the next reads.
                // Without it the compiler puts a full LDS wait after those
                // reads, since it counts the direct-to-LDS loads of step 0 as
                // LDS accesses that may complete out of order.
                if constexpr (EARLY || WEAVE)
                    if (step > 0)
                        wait_lds_only();
                if (step % 2 == 0)
                    read_frags<BM, BKB, TM, TN>(S, step + 1, wm0, wn0, lane, fa1, fb1);
                else
                    read_frags<BM, BKB, TM, TN>(S, step + 1, wm0, wn0, lane, fa0, fb0);
                if constexpr (EARLY) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (!SPREAD && step == 0)
                        dma_entry(e + NS - 1);   // interleaved with step 0's MFMAs
                }
                if constexpr (WEAVE)
                    if (step == 0)
                        dma_entry(e + NS - 1);
                if (step % 2 == 0)
                    mfma_step<P, TM, TN, 0, TM * TN, TRANS>(fa0, fb0, acc);
                else
                    mfma_step<P, TM, TN, 0, TM * TN, TRANS>(fa1, fb1, acc);
                if constexpr (WEAVE) {
                    if (step == 0)
                        weave_order<true, TM * TN>();
                    else
                        weave_order<false, TM * TN>();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SPREAD)
                dma_step(e + NS - 1, STEPS - 1);
            mfma_step<P, TM, TN, 0, KA, TRANS>(fa1, fb1, acc);
            __builtin_amdgcn_sched_barrier(0);
            stage_regs(e + NS - 1);   // (VGPR-staged variant only) into the free stage
            wait_vm_lds<(NS - 2) * NL>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_frags<BM, BKB, TM, TN>(Snext, 0, wm0, wn0, lane, fa0, fb0);
            if constexpr (EARLY)
                __builtin_amdgcn_sched_barrier(0);
            mfma_step<P, TM, TN, KA, NMF, TRANS>(fa1, fb1, acc);
            if constexpr (WEAVE)
                weave_order<false, NMF - KA>();
            __builtin_amdgcn_sched_barrier(0);
        }
        // the last entries' dummy loads must land before the ring is reused
        wait_vm_lds<0>();
    }

    // Output of a finished tile from this loop's accumulators: C through LDS
    // with 16-byte stores for the transposed layout (every wavefront must be
    // past its last fragment read and its loads landed before the ring is
    // reused: one barrier), otherwise as epilogue_direct.
    static __device__ __forceinline__ void epilogue(const GemmProblem &p, uint8_t *smem, int row0,
                                                    int col0, int tid, int lane, int wave,
                                                    const acc_t (&acc)[TM][TN]) {
        if constexpr (TRANS && P == PREC_W4A4) {
            const int wm0 = (wave / WGN) * WTM;
            const int wn0 = (wave % WGN) * WTN;
            float *fac = reinterpret_cast<float *>(smem + LDS_BYTES - FACB);
            stage_factors<BM, BN, NT>(p, row0, col0, tid, fac);   // (barriers before and after)
            store_tile_lds_w4a4<TM, TN, RP>(p, smem + wave * REGION, row0 + wm0, col0 + wn0, lane, acc,
                                            fac + wm0, fac + BM + wn0, fac + BM + BN + wn0);
        } else if constexpr (TRANS) {
            const int wm0 = (wave / WGN) * WTM;
            const int wn0 = (wave % WGN) * WTN;
            __syncthreads();
            store_tile_lds<P, TM, TN, RP>(p, smem + wave * (LDS_BYTES / NW), row0 + wm0, col0 + wn0, lane,
                                          acc);
        } else {
            epilogue_direct(p, smem, row0, col0, tid, lane, wave, acc);
        }
    }

    // Output of a finished tile whose accumulators hold C blocks directly
    // (not transposed): C for the plain GEMMs; for W4A4 the scale epilogue
    // with the factors staged in the (then free) LDS ring.
    static __device__ __forceinline__ void epilogue_direct(const GemmProblem &p, uint8_t *smem, int row0,
                                                           int col0, int tid, int lane, int wave,
                                                           const acc_t (&acc)[TM][TN]) {
        const int wm0 = (wave / WGN) * WTM;
        const int wn0 = (wave % WGN) * WTN;
        if constexpr (P == PREC_W4A4) {
            static_assert((BM + 2 * BN) * 4 <= LDS_BYTES, "factor staging fits the ring");
            float *fac = reinterpret_cast<float *>(smem);
            stage_factors<BM, BN, NT>(p, row0, col0, tid, fac);
            store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc, fac + wm0, fac + BM + wn0,
                                  fac + BM + BN + wn0);
        } else {
            store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc);
        }
    }
};

// Data-parallel kernel: one output tile per workgroup, all of K.
template <int P, int BM, int BN, int BKB, int WGM, int WGN, int NS, int VAR>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tile_kernel(GemmProblem p, int tiles_m,
                                                                   int tiles_n) {
    typedef RingTile<P, BM, BN, BKB, WGM, WGN, NS, VAR> RT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[RT::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // made explicitly uniform so the per-wavefront LDS bases live in scalar
    // registers: the DMA destinations then need no per-copy readfirstlane
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int KT = (int)((p.kbytes + BKB - 1) / BKB);

    typename RT::acc_t acc[RT::TM][RT::TN];
    RT::mainloop(p, smem, row0, col0, 0, KT, tid, lane, wave, acc);
    RT::epilogue(p, smem, row0, col0, tid, lane, wave, acc);
}

// Direct-to-register variant of the 256 x 256 tile: A goes through the LDS
// ring as in RingTile, B does not touch LDS. Each wavefront loads the B
// fragments of its 128 columns straight from global memory into registers,
// one stage ahead, in the MFMA operand layout (lane l holds column l % 32 of
// a 32-column block). That halves the LDS traffic per MFMA (fragment reads
// and DMA writes both carry A only) at the price of reading every B row from
// L2 twice per workgroup (the two wavefronts of a column pair).
//
// K order inside a 128-byte stage: lane group g = l / 32 takes chunk 4g + s
// at k-step s, so one lane's B bytes over the stage are 64 contiguous bytes
// of its row. A's fragment reads use the same chunk, so both operands present
// the same k to each MFMA product and the dot product is unchanged.
//
// Iteration e (stage e in LDS slot e % NS, B registers hold stage e): the
// direct-to-LDS loads of A entry e + NS - 1 into the slot freed by entry
// e - 1; per k-step s the A fragment reads of step s + 1, the MFMAs of step
// s, then the B loads of step s of stage e + 1 into the registers those
// MFMAs just consumed. Entries past the last K tile re-read it (unused), so
// every iteration issues the same 8 + 16 loads and the wait for A entry
// e + 1 is a constant vmcnt. K must be a whole number of stages.
//
// Measured on MI355X slower than the ring kernel it varies (INT8 8192^3:
// 1630 vs 2205 TOP/s, FP16 859 vs 1185 TFLOP/s, INT4 2452 vs 2582 TOP/s),
// with the same result for a 3-stage A ring: one B load instruction touches
// 32 rows (the MFMA layout puts one row per lane), 32 cache lines for 1 KiB,
// where a direct-to-LDS load touches 8, and the compute unit's load path,
// not LDS, sets the pace. Kept as an ablation configuration
// (CFG_256x256_DTV, built with NS = 2).
// vmcnt wait that leaves lgkmcnt (LDS reads in flight) alone.
template <int VM>
__device__ __forceinline__ void wait_vm_only() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}

// A 16-byte global load into a VGPR quad through inline assembly (uniform
// 64-bit base in SGPRs, 32-bit lane offset), which the compiler does not
// count: its analysis of loop-carried register loads falls back to waiting
// for every load in flight, including the A tile just issued. The register
// is tied in and out, so the load writes the quad that holds the variable;
// the value may be read only after a wait that covers the load and
// untracked_ready16().
__device__ __forceinline__ void load16_untracked(i32x4 &v, uint32_t voff, const void *sbase) {
    asm volatile("global_load_dwordx4 %0, %1, %2" : "+v"(v) : "v"(voff), "s"(sbase));
}
__device__ __forceinline__ void untracked_ready16(i32x4 &v) { asm volatile("" : "+v"(v)); }

template <int P, int NS>
struct DtvTile {
    static constexpr int BM = 256, BN = 256, BKB = 128, WGM = 2, WGN = 2;
    static constexpr int NT = 256, WTM = 128, WTN = 128, TM = 4, TN = 4;
    static constexpr int CPR = BKB / 16, RS = NT / CPR, NLA = BM / RS;   // 8 A loads per thread
    static constexpr int STEPS = CPR / 2;                                 // 4 k-steps per stage
    static constexpr int NLB = STEPS * TN;                                // 16 B loads per lane
    static constexpr int STAGE = BM * BKB;
    static constexpr int LDS_BYTES = NS * STAGE;
    // vmcnt when A entry e + 1 must have landed (end of iteration e): the B
    // loads of steps 0..2 of this iteration, plus for NS = 3 everything issued
    // since entry e + 1 at the top of iteration e - 1.
    static constexpr int WAIT_A = 3 * TN + (NS - 2) * (NLA + NLB);
    // vmcnt before the MFMAs of a k-step: its B registers were loaded one
    // stage earlier; younger are the other three steps' B loads and this
    // iteration's A loads.
    static constexpr int WAIT_B = 3 * TN + NLA;
    static_assert(NS == 2 || NS == 3, "vmcnt of the A wait must fit 6 bits");
    static_assert(WAIT_A < 64 && 8 * (NS - 2) + NLB < 64, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KiB");
    typedef typename AccOf<P>::type acc_t;

    static __device__ __forceinline__ void read_a(const uint8_t *As, int step, int wm0, int lane,
                                                  i32x4 (&a)[TM]) {
        const int c = 4 * (lane >> 5) + step;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm0 + i * 32 + (lane & 31);
            a[i] = *reinterpret_cast<const i32x4 *>(As + r * BKB + ((c ^ swz<CPR>(r)) * 16));
        }
    }

    static __device__ __forceinline__ void mainloop(const GemmProblem &p, uint8_t *smem, int row0,
                                                    int col0, int tid, int lane, int wave,
                                                    acc_t (&acc)[TM][TN]) {
        const int wm0 = (wave / WGN) * WTM;
        const int wn0 = (wave % WGN) * WTN;
        const int KT = (int)(p.kbytes / BKB);

        // A: thread tid loads rows r0 + RS * i, chunk slot tid % CPR
        const int r0 = tid / CPR;
        const int cg = (tid % CPR) ^ swz<CPR>(r0);
        const uint8_t *Ab = p.A + (int64_t)row0 * p.lda_b;
        const int a_rows = p.M - row0;
        uint32_t aoff[NLA];
#pragma unroll
        for (int i = 0; i < NLA; ++i) {
            int r = r0 + i * RS;
            r = r < a_rows ? r : a_rows - 1;   // clamped rows feed outputs never stored
            aoff[i] = (uint32_t)r * (uint32_t)p.lda_b + cg * 16;
        }
        const int wrow = wave * (64 / CPR);
        // B: lane l of block j reads row wn0 + 32 j + l % 32, bytes 64 (l / 32) ...
        const uint8_t *Bb = p.B + (int64_t)col0 * p.ldb_b;
        const int b_rows = p.N - col0;
        uint32_t boff[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            int r = wn0 + j * 32 + (lane & 31);
            r = r < b_rows ? r : b_rows - 1;
            boff[j] = (uint32_t)r * (uint32_t)p.ldb_b + 64 * (lane >> 5);
        }

        auto dma_a = [&](int e) {
            const int kt = e < KT - 1 ? e : KT - 1;
            uint8_t *S = smem + (e % NS) * STAGE;
#pragma unroll
            for (int i = 0; i < NLA; ++i)
                dma16_cp<0>(Ab + (int64_t)kt * BKB + aoff[i], S + (wrow + i * RS) * BKB);
        };
        // B registers of the current stage; load_b(e, s) refills breg[s] with
        // step s of stage e. The loads are untracked (see load16_untracked),
        // so the consumers wait with wait_vm_only<WAIT_B>() and b_ready().
        i32x4 breg[STEPS][TN];
        auto load_b = [&](int e, int s) {
            const int kt = e < KT - 1 ? e : KT - 1;
            const uint8_t *src = Bb + (int64_t)kt * BKB + 16 * s;   // uniform
#pragma unroll
            for (int j = 0; j < TN; ++j)
                load16_untracked(breg[s][j], boff[j], src);
        };
        auto b_ready = [&](int s) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                untracked_ready16(breg[s][j]);
        };

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = acc_t{};
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                breg[s][j] = i32x4{0, 0, 0, 0};

        i32x4 fa0[TM], fa1[TM];
#pragma unroll
        for (int e = 0; e < NS - 1; ++e)
            dma_a(e);
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            load_b(0, s);
        wait_vm_lds<NLA * (NS - 2) + NLB>();   // A entry 0
        lds_barrier();
        read_a(smem, 0, wm0, lane, fa0);

        constexpr int NMF = TM * TN;
        constexpr int KA = NMF / 4;
        for (int e = 0; e < KT; ++e) {
            const uint8_t *S = smem + (e % NS) * STAGE;
            const uint8_t *Snext = smem + ((e + 1) % NS) * STAGE;
            __builtin_amdgcn_sched_barrier(0);
            dma_a(e + NS - 1);
#pragma unroll
            for (int step = 0; step < STEPS - 1; ++step) {
                if (step % 2 == 0)
                    read_a(S, step + 1, wm0, lane, fa1);
                else
                    read_a(S, step + 1, wm0, lane, fa0);
                wait_vm_only<WAIT_B>();
                b_ready(step);
                if (step % 2 == 0)
                    mfma_step<P, TM, TN>(fa0, breg[step], acc);
                else
                    mfma_step<P, TM, TN>(fa1, breg[step], acc);
                load_b(e + 1, step);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vm_only<WAIT_B>();
            b_ready(STEPS - 1);
            mfma_step<P, TM, TN, 0, KA>(fa1, breg[STEPS - 1], acc);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_lds<WAIT_A>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_a(Snext, 0, wm0, lane, fa0);
            mfma_step<P, TM, TN, KA, NMF>(fa1, breg[STEPS - 1], acc);
            load_b(e + 1, STEPS - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The last entries' dummy loads must land before the ring is reused,
        // and the last B loads before their registers are: the registers stay
        // live up to here, so the compiler cannot hand them to the epilogue
        // while those loads are still in flight.
        wait_vm_lds<0>();
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            b_ready(s);
    }
};

// Data-parallel kernel of DtvTile (K a whole number of 128-byte stages).
template <int P, int NS>
__global__ __launch_bounds__(256) void gemm_dtv_kernel(GemmProblem p, int tiles_m, int tiles_n) {
    typedef DtvTile<P, NS> DT;
    typedef RingTile<P, 256, 256, 128, 2, 2, 2> RT;   // same wavefront tiles: its direct epilogue
    static_assert(RT::LDS_BYTES >= (256 + 2 * 256) * 4, "epilogue staging");
    __shared__ __attribute__((aligned(16))) uint8_t smem[DT::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * 256, col0 = tn * 256;

    typename DT::acc_t acc[DT::TM][DT::TN];
    DT::mainloop(p, smem, row0, col0, tid, lane, wave, acc);
    RT::epilogue_direct(p, smem, row0, col0, tid, lane, wave, acc);
}

// Ping-pong kernel for the 256 x 256 tile (data-parallel, K a multiple of
// the 128-byte stage, at least two stages). Eight wavefronts, two per SIMD,
// in two groups of four (wavefronts q and q + 4 share SIMD q) that run the
// same loop one phase apart. A phase ends at a workgroup barrier; in each
// phase one group issues the MFMAs of two k-steps from fragments that are
// already in its registers, while the other group reads the fragments of its
// next two k-steps from LDS and issues its share of the direct-to-LDS loads.
// A wavefront's fragment reads are then covered by its SIMD partner's MFMAs
// instead of its own. The price is 1.5x the fragment bytes per MFMA (128 x 64
// wavefront tiles instead of 128 x 128): four wavefronts reading 12 KiB each
// per phase need about as long as the phase's MFMAs, so on MI355X the memory
// half, not the matrix unit, sets the pace. Measured slower than the
// four-wavefront ring kernel except for INT8 at 4096; kept as an ablation
// configuration (the override index CFG_256x256_PP).
//
// Wavefront (g, q): rows [128 (q / 2), +128), columns [128 (q % 2) + 64 g,
// +64) of the tile. Stage e (entry e of K) lives in LDS stage e % 2 and is
// read in the group's phase pairs 2e and 2e + 1. Entry e + 1 (e >= 1) is
// loaded during pair 2e into the stage that entry e - 1 used (free: the last
// read of it ended before the barrier that opens pair 2e), and every
// wavefront waits for its own loads at the end of the memory half of pair
// 2e + 1, so the barrier that follows publishes the entry to both groups
// before pair 2e + 2.
template <int P>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmProblem p, int tiles_m, int tiles_n) {
    constexpr int BM = 256, BN = 256, BKB = 128, NS = 2, NT = 512;
    constexpr int CPR = BKB / 16;                      // 16-byte chunks per LDS row
    constexpr int RS = NT / CPR;                       // rows per load round
    constexpr int A_PER_T = BM / RS, B_PER_T = BN / RS;
    constexpr int NL = A_PER_T + B_PER_T;              // loads per thread per stage
    constexpr int STAGE = (BM + BN) * BKB;
    constexpr int PS = 2;                              // k-steps per phase
    constexpr int PAIRS = (CPR / 2) / PS;              // phases per stage and group
    constexpr int TM = 4, TN = 2;                      // 128 x 64 per wavefront
    static_assert(PAIRS == 2, "the load schedule assumes two phases per stage");
    typedef typename AccOf<P>::type acc_t;
    __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm0 = (q >> 1) * 128, wn0 = (q & 1) * 128 + grp * 64;

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int KT = (int)(p.kbytes / BKB);

    // direct-to-LDS addressing as in RingTile: thread rows r0 + i * RS, the
    // global chunk that the swizzle puts in the thread's LDS slot
    const int r0 = tid / CPR;
    const int cg = (tid % CPR) ^ swz<CPR>(r0);
    const uint8_t *Ab = p.A + (int64_t)row0 * p.lda_b;
    const uint8_t *Bb = p.B + (int64_t)col0 * p.ldb_b;
    const int a_rows = p.M - row0, b_rows = p.N - col0;
    uint32_t off[NL];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        int r = r0 + i * RS;
        r = r < a_rows ? r : a_rows - 1;   // clamped rows feed outputs never stored
        off[i] = (uint32_t)r * (uint32_t)p.lda_b + cg * 16;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        int r = r0 + i * RS;
        r = r < b_rows ? r : b_rows - 1;
        off[A_PER_T + i] = (uint32_t)r * (uint32_t)p.ldb_b + cg * 16;
    }
    const int wrow = wave * (64 / CPR);
    auto dma_entry = [&](int kt) {
        const uint8_t *a = Ab + (int64_t)kt * BKB;
        const uint8_t *b = Bb + (int64_t)kt * BKB;
        uint8_t *S = smem + (kt % NS) * STAGE + wrow * BKB;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            dma16(a + off[i], S + i * RS * BKB);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i)
            dma16(b + off[A_PER_T + i], S + BM * BKB + i * RS * BKB);
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = acc_t{};
    i32x4 fa[PS][TM], fb[PS][TN];

    dma_entry(0);
    dma_entry(1);
    wait_vm_lds<0>();
    lds_barrier();
    if (grp == 1)
        lds_barrier();   // group 1 runs one phase behind group 0

    const int NPAIR = KT * PAIRS;
    for (int j = 0; j < NPAIR; ++j) {
        const int e = j / PAIRS, h = j % PAIRS;
        const uint8_t *S = smem + (e % NS) * STAGE;
        // memory half: fragments of k-steps h PS .. h PS + PS - 1 of entry e
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < PS; ++s)
            read_frags<BM, BKB, TM, TN>(S, h * PS + s, wm0, wn0, lane, fa[s], fb[s]);
        if (h == 0 && e >= 1 && e + 1 < KT)
            dma_entry(e + 1);
        if (h == PAIRS - 1)
            wait_vm_lds<0>();    // this wavefront's loads of entry e + 1 have landed
        else
            wait_vm_lds<63>();   // fragment reads only
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        // compute half
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < PS; ++s)
            mfma_step<P, TM, TN>(fa[s], fb[s], acc);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
    }
    if (grp == 0)
        lds_barrier();   // same barrier count in both groups

    store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc);
}

// Stream-K partial accumulators: 16-byte loads and stores that are coherent
// across the XCDs' L2 caches (sc1: written through, read past a stale line),
// so that no cache-wide write-back or invalidation is needed.
__device__ __forceinline__ void sk_store16(__amdgpu_buffer_rsrc_t r, int off, i32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16);
}
__device__ __forceinline__ i32x4 sk_load16(__amdgpu_buffer_rsrc_t r, int off) {
    // the builtin's own 16-byte vector type; converting it implicitly to
    // i32x4 would narrow the load to its first dword
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
    return __builtin_bit_cast(i32x4, v);
}

// Workgroup whose stream-K range holds iteration x (ranges [w I / G, (w+1) I / G)).
__device__ __forceinline__ int sk_owner(int64_t x, int64_t iters, int grid) {
    return (int)(((x + 1) * grid - 1) / iters);
}

// Stream-K kernel ("Stream-K" work decomposition, the persistent tile
// scheduling that the L4 study names as next step): a persistent grid of G
// workgroups first runs tiles [0, tiles_dp) whole (round-robin), then splits
// the K iterations of the remaining tiles evenly: workgroup w runs iterations
// [w I / G, (w+1) I / G), tile by tile. A tile whose iterations span several
// workgroups is finished by the last of them to arrive: each contributor
// stores its partial accumulators (coherent stores), waits for them to
// complete and increments the tile's counter; the one that sees all others
// done sums the contributions in workgroup order (its own from registers),
// writes the output and resets the counter to zero. Nobody waits on another
// workgroup, and the summation order does not depend on arrival order.
template <int P, int BM, int BN, int BKB, int WGM, int WGN, int NS, int VAR>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tile_sk_kernel(GemmProblem p, int tiles_m,
                                                                      int tiles_n, StreamKArgs sk) {
    typedef RingTile<P, BM, BN, BKB, WGM, WGN, NS, VAR> RT;
    typedef typename RT::acc_t acc_t;
    constexpr int TM = RT::TM, TN = RT::TN, NT = RT::NT;
    constexpr int SLOT = BM * BN * 4;   // bytes of one partial tile
    typedef typename AccOf<P>::elem elem4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint8_t smem[RT::LDS_BYTES];
    __shared__ int sk_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x;
    const int w = xcd_logical(blockIdx.x, G);
    const int KT = (int)((p.kbytes + BKB - 1) / BKB);

    acc_t acc[TM][TN];
    int tm, tn;
    for (int t = w; t < sk.tiles_dp; t += G) {
        tile_raster(t, tiles_m, tiles_n, tm, tn);
        RT::mainloop(p, smem, tm * BM, tn * BN, 0, KT, tid, lane, wave, acc);
        RT::epilogue(p, smem, tm * BM, tn * BN, tid, lane, wave, acc);
        __syncthreads();   // the ring is free again
    }

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(sk.partial, 0, sk.partial_bytes, 0x00020000);
    const int64_t I = sk.iters;
    const int64_t beg = I * w / G, end = I * (w + 1) / G;
    for (int64_t it = beg; it < end;) {
        const int tl = (int)(it / KT);
        const int e0 = (int)(it - (int64_t)tl * KT);
        const int e1 = (int)((int64_t)KT - e0 < end - it ? KT : e0 + (end - it));
        tile_raster(sk.tiles_dp + tl, tiles_m, tiles_n, tm, tn);
        const int row0 = tm * BM, col0 = tn * BN;
        RT::mainloop(p, smem, row0, col0, e0, e1, tid, lane, wave, acc);
        bool finish = e0 == 0 && e1 == KT;
        if (!finish) {
            const int64_t t0 = (int64_t)tl * KT;
            const int w_lo = sk_owner(t0, I, G), w_hi = sk_owner(t0 + KT - 1, I, G);
            const int n = w_hi - w_lo + 1;
            // slot 0: the tile where a workgroup's range starts (floor(I v / G)
            // >= t0, i.e. I v >= t0 G); slot 1: the other one
            auto slot_off = [&](int v) {
                const bool first = I * v >= t0 * G;
                return (2 * v + (first ? 0 : 1)) * SLOT;
            };
            // Ordering: each contributor's partial stores complete (and are
            // released at agent scope by the increment) before its counter
            // increment; the finisher's acquire (this load, or the
            // increment that makes it the last) and the agent-scope acquire
            // fence of every thread below order its partial loads after them.
            if (tid == 0)
                sk_flag = __hip_atomic_load(sk.flags + tl, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            finish = sk_flag == n - 1;   // every other contributor is done already
            if (!finish) {
                const int base = slot_off(w);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            // whole vectors are bit-cast (never a vector element)
                            const elem4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                             acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            sk_store16(rs, base + (((i * TN + j) * 4 + q) * NT + tid) * 16,
                                       __builtin_bit_cast(i32x4, v));
                        }
                // stores complete (written through) before the counter moves
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0);
                asm volatile("" ::: "memory");
                __syncthreads();
                if (tid == 0)
                    sk_flag = __hip_atomic_fetch_add(sk.flags + tl, 1, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                finish = sk_flag == n - 1;
            }
            if (finish) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                // sum of the contributions in workgroup order
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc_t sum = acc[i][j];
                        for (int v = w_lo; v <= w_hi; ++v) {
                            acc_t c = acc[i][j];
                            if (v != w) {
                                const int base = slot_off(v);
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const elem4 x = __builtin_bit_cast(
                                        elem4, sk_load16(rs, base + (((i * TN + j) * 4 + q) * NT + tid) * 16));
#pragma unroll
                                    for (int d = 0; d < 4; ++d)
                                        c[4 * q + d] = x[d];
                                }
                            }
                            sum = v == w_lo ? c : sum + c;
                        }
                        acc[i][j] = sum;
                    }
                if (tid == 0)
                    __hip_atomic_store(sk.flags + tl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (finish)
            RT::epilogue(p, smem, row0, col0, tid, lane, wave, acc);
        __syncthreads();   // the ring (and sk_flag) are free again
        it += e1 - e0;
    }
}

// Operands without 16-byte row alignment (or with rows too long for 32-bit
// offsets, or K shorter than one tile): byte-gather loads, 64-bit
// addressing, single prefetch.
template <int P, int BM, int BN, int BKB, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tile_generic_kernel(GemmProblem p,
                                                                           int tiles_m,
                                                                           int tiles_n) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int CPR = BKB / 16;
    constexpr int RS = NT / CPR;
    constexpr int A_PER_T = BM / RS, B_PER_T = BN / RS;
    constexpr int NL = A_PER_T + B_PER_T;
    constexpr int STAGE = (BM + BN) * BKB;
    static_assert(RS % 16 == 0 && BM % RS == 0 && BN % RS == 0, "staging must divide evenly");
    typedef typename AccOf<P>::type acc_t;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WGN) * WTM, wn0 = (wave % WGN) * WTN;
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int64_t kbytes = p.kbytes;
    const int KT = (int)((kbytes + BKB - 1) / BKB);
    const int c = tid % CPR, r0 = tid / CPR;
    const int lds0 = r0 * BKB + ((c ^ swz<CPR>(r0)) * 16);

    auto load = [&](int kt, i32x4 *R) {
        const int64_t k = (int64_t)kt * BKB + c * 16;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const bool isA = i < A_PER_T;
            const int gr = (isA ? row0 : col0) + r0 + (isA ? i : i - A_PER_T) * RS;
            const bool ok = gr < (isA ? p.M : p.N);
            const uint8_t *row = (isA ? p.A : p.B) + (int64_t)(ok ? gr : 0) * (isA ? p.lda_b : p.ldb_b);
            R[i] = load_chunk_bytes(row, k, kbytes, ok);
        }
    };
    auto store = [&](int stage, const i32x4 *R) {
        uint8_t *S = smem + stage * STAGE + lds0;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            *reinterpret_cast<i32x4 *>(S + i * RS * BKB) = R[i];
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i)
            *reinterpret_cast<i32x4 *>(S + BM * BKB + i * RS * BKB) = R[A_PER_T + i];
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = acc_t{};
    i32x4 R[NL];
    if (KT > 0) {
        load(0, R);
        store(0, R);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load(kt + 1, R);
#pragma unroll
        for (int step = 0; step < CPR / 2; ++step) {
            i32x4 fa[TM], fb[TN];
            read_frags<BM, BKB, TM, TN>(smem + cur * STAGE, step, wm0, wn0, lane, fa, fb);
            mfma_step<P, TM, TN>(fa, fb, acc);
        }
        if (kt + 1 < KT)
            store(cur ^ 1, R);
        __syncthreads();
    }
    if constexpr (P == PREC_W4A4) {
        static_assert((BM + 2 * BN) * 4 <= 2 * STAGE, "factor staging fits the buffers");
        float *fac = reinterpret_cast<float *>(smem);
        stage_factors<BM, BN, NT>(p, row0, col0, tid, fac);
        store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc, fac + wm0, fac + BM + wn0,
                              fac + BM + BN + wn0);
    } else {
        store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc);
    }
}

// Transposed-B control (the L4 study's ablation of the B operand's layout):
// B is stored K x N, each row of B^T holding the N values of one k. For
// INT4 two n share a byte (the low nibble holds the even n), since n is the
// contiguous dimension. The kernel is the VGPR-staged two-buffer tile
// kernel (as gemm_tile_generic_kernel, 16-byte aligned rows) with one change:
// B's 16-byte chunks, coalesced along n, are written into the same
// [n][k]-ordered, swizzled LDS layout as the N x K path, element by element
// (INT4: a byte from the nibbles of two rows), so the fragment reads, the
// MFMAs and the epilogue are unchanged. The transposition costs one LDS
// write per element instead of one per 16 bytes.
template <int P>
__global__ __launch_bounds__(256) void gemm_tile_kn_kernel(GemmProblem p, int tiles_m, int tiles_n) {
    constexpr int BM = 256, BN = 256, BKB = 128, WGN = 2;
    constexpr int NT = 256, WTM = 128, WTN = 128, TM = 4, TN = 4;
    constexpr int CPR = BKB / 16, RS = NT / CPR, A_PER_T = BM / RS;
    constexpr int STAGE = (BM + BN) * BKB;
    // B^T staging: chunks of 16 bytes along n. CPB chunks per B^T row of the
    // tile; INT4 loads the chunks of rows 2 kp and 2 kp + 1 together.
    constexpr int CPB = P == PREC_F16 ? 32 : (P == PREC_I8 ? 16 : 8);
    constexpr int NPC = P == PREC_F16 ? 8 : (P == PREC_I8 ? 16 : 32);   // n per chunk
    constexpr int ROWS = P == PREC_I4 ? 2 : 1;                          // B^T rows per item
    constexpr int KPS = P == PREC_F16 ? 64 : (P == PREC_I8 ? 128 : 256);    // k per stage
    constexpr int ITEMS = KPS / ROWS * CPB / NT;
    static_assert(P != PREC_W4A4, "no scale epilogue on this path");
    static_assert(ITEMS * ROWS == 8, "8 B chunks per thread per stage");
    typedef typename AccOf<P>::type acc_t;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WGN) * WTM, wn0 = (wave % WGN) * WTN;
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int64_t kbytes = p.kbytes;
    // k values (INT4: nibbles) per row of A, and the bytes of one B^T row
    const int64_t K = P == PREC_F16 ? kbytes / 2 : (P == PREC_I8 ? kbytes : 2 * kbytes);
    const int64_t nbytes = P == PREC_F16 ? 2 * (int64_t)p.N : (P == PREC_I8 ? p.N : ((int64_t)p.N + 1) / 2);
    const int KT = (int)((kbytes + BKB - 1) / BKB);
    const int c = tid % CPR, r0 = tid / CPR;
    const int lds0 = r0 * BKB + ((c ^ swz<CPR>(r0)) * 16);

    i32x4 RA[A_PER_T], RB[8];
    auto load = [&](int kt) {
        const int64_t ka = (int64_t)kt * BKB + c * 16;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int gr = row0 + r0 + i * RS;
            const bool ok = gr < p.M;
            RA[i] = load_chunk_masked(p.A + (int64_t)(ok ? gr : 0) * p.lda_b, ka, kbytes, ok);
        }
        const int64_t k0 = (int64_t)kt * KPS;   // the stage's first B^T row
        const int64_t colb = P == PREC_F16 ? 2 * (int64_t)col0 : (P == PREC_I8 ? col0 : col0 / 2);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int q = tid + i * NT;
            const int kl = (q / CPB) * ROWS, nc = q % CPB;
            const int64_t off = colb + nc * 16;
#pragma unroll
            for (int h = 0; h < ROWS; ++h) {
                const int64_t k = k0 + kl + h;
                const bool ok = k < K;
                RB[i * ROWS + h] = load_chunk_masked(p.B + (ok ? k : 0) * p.ldb_b, off, nbytes, ok);
            }
        }
    };
    auto store = [&](int stage) {
        uint8_t *S = smem + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            *reinterpret_cast<i32x4 *>(S + lds0 + i * RS * BKB) = RA[i];
        uint8_t *SB = S + BM * BKB;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int q = tid + i * NT;
            const int kl = (q / CPB) * ROWS, nc = q % CPB;
            // byte of the [n][k] row that this item's k lands in
            const int kb = P == PREC_F16 ? 2 * kl : (P == PREC_I8 ? kl : kl / 2);
            const int kc = kb >> 4, kw = kb & 15;
#pragma unroll
            for (int e = 0; e < NPC; ++e) {
                const int r = nc * NPC + e;
                uint8_t *dst = SB + r * BKB + ((kc ^ swz<CPR>(r)) << 4) + kw;
                if constexpr (P == PREC_F16) {
                    const uint32_t w = (uint32_t)RB[i][e >> 1];
                    *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(w >> (16 * (e & 1)));
                } else if constexpr (P == PREC_I8) {
                    *dst = (uint8_t)((uint32_t)RB[i][e >> 2] >> (8 * (e & 3)));
                } else {
                    // nibble e of the chunks of rows k (low) and k + 1 (high)
                    const uint32_t lo = (uint32_t)RB[2 * i][e >> 3] >> (4 * (e & 7));
                    const uint32_t hi = (uint32_t)RB[2 * i + 1][e >> 3] >> (4 * (e & 7));
                    *dst = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
                }
            }
        }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = acc_t{};
    if (KT > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load(kt + 1);
#pragma unroll
        for (int step = 0; step < CPR / 2; ++step) {
            i32x4 fa[TM], fb[TN];
            read_frags<BM, BKB, TM, TN>(smem + cur * STAGE, step, wm0, wn0, lane, fa, fb);
            mfma_step<P, TM, TN>(fa, fb, acc);
        }
        if (kt + 1 < KT)
            store(cur ^ 1);
        __syncthreads();
    }
    store_tile<P, TM, TN>(p, row0 + wm0, col0 + wn0, lane, acc);
}

// ------------------------------------------------------------------ launch

// BM x BN tile, BKB bytes of K per stage, blocks that one compute unit holds
// at once (LDS: NS * (BM + BN) * BKB bytes each, 160 KiB per CU).
struct CfgShape { int BM, BN, BKB, per_cu; const char *name; };
static const CfgShape kCfg[CFG_COUNT] = {
    {256, 256, 64, 1, "256x256_bk64_ring4"},
    {128, 128, 64, 2, "128x128_bk64_ring4"},
    {64, 64, 128, 3, "64x64_bk128_ring3"},
    {256, 128, 128, 1, "256x128_bk128_ring3"},
    {256, 256, 128, 1, "256x256_bk128_ring2"},
    {128, 256, 128, 1, "128x256_bk128_ring3"},
    {128, 128, 128, 1, "128x128_bk128_ring4"},
    {256, 256, 128, 1, "256x256_bk128_ring2_w8"},
    {256, 256, 64, 1, "256x256_bk64_ring4_w8"},
    {256, 128, 64, 2, "256x128_bk64_ring3_2blk"},
    {128, 128, 128, 2, "128x128_bk128_ring2_2blk"},
    {128, 256, 64, 2, "128x256_bk64_ring3_2blk"},
    {256, 256, 128, 1, "256x256_bk128_pingpong"},
    {256, 256, 128, 1, "256x256_bk128_ring2_split_loaders"},
    {256, 256, 128, 1, "256x256_bk128_ring2_nt"},
    {256, 256, 128, 1, "256x256_bk128_ring2_sc1"},
    {256, 256, 128, 1, "256x256_bk128_ring2_vgpr_staged"},
    {256, 256, 128, 1, "256x256_bk128_ring2_spread_loads"},
    {256, 256, 128, 1, "256x256_bk128_a_ring2_b_direct"},
    {256, 256, 128, 1, "256x256_bk128_ring2_sc0"},
    {256, 256, 128, 1, "256x256_bk128_ring2_early_frag_reads"},
    {256, 256, 128, 1, "256x256_bk128_ring2_woven_frag_reads"},
    {64, 64, 128, 1, "64x64_bk128_ring8"},
};

const char *tile_cfg_name(int cfg) {
    return (cfg >= 0 && cfg < CFG_COUNT) ? kCfg[cfg].name : "invalid";
}

int choose_tile_cfg(int prec, int64_t M, int64_t N, int64_t kbytes, int cu_count) {
    auto tiles = [&](int c) {
        return ((M + kCfg[c].BM - 1) / kCfg[c].BM) * ((N + kCfg[c].BN - 1) / kCfg[c].BN);
    };
    // Largest tile that still gives every compute unit a workgroup (measured
    // on MI355X: the 256x256 tile with a 128-byte K depth is the fastest once
    // the grid fills the chip).
    if (tiles(CFG_256x256_BK128) >= cu_count)
        return CFG_256x256_BK128;
    if (tiles(CFG_256x128) >= cu_count)
        return CFG_256x128;
    if (tiles(CFG_128x128_BK128) >= cu_count / 2)
        return CFG_128x128_BK128;
    // FP16 with at least 16 K stages: the 8-stage ring keeps most of the
    // short K loop in flight (1024^3: 8.0 vs 8.5 us); INT8 / INT4 and FP16 at
    // 512^3 measured 2-4 % slower with it (their loops are 4-8 stages)
    if (prec == 0 && kbytes >= 16 * 128)
        return CFG_64x64_DEEP;
    return CFG_64x64;
}

StreamKPlan plan_stream_k(int cfg, int64_t M, int64_t N, int64_t kbytes, int cu_count,
                          int64_t partial_bytes, int flag_count, int mode) {
    StreamKPlan pl = {0, 0, 0, 0};
    if (mode == SK_MODE_OFF || cfg < 0 || cfg >= CFG_COUNT || cu_count < 1)
        return pl;
    const CfgShape &c = kCfg[cfg];
    const int64_t KT = (kbytes + c.BKB - 1) / c.BKB;
    if (kbytes < c.BKB || KT < 2)   // the generic kernel, or nothing to split
        return pl;
    const int64_t T = ((M + c.BM - 1) / c.BM) * ((N + c.BN - 1) / c.BN);
    const int64_t G = (int64_t)cu_count * c.per_cu;   // workgroups resident at once
    if (mode == SK_MODE_PERSIST) {
        if (T > INT32_MAX)
            return pl;
        pl.grid = (int)(T < G ? T : G);
        pl.tiles_dp = (int)T;
        return pl;   // sk_tiles = iters = 0
    }
    const int64_t full = T / G, rem = T % G;
    if (rem == 0)
        return pl;   // whole waves: nothing to balance
    if (mode == SK_MODE_AUTO) {
        // A split tile's partial sums make a round trip through memory
        // (written through past the XCD's L2, read back by the finishing
        // workgroup). Measured on MI355X that costs more than the idle tail
        // of a short last wave (INT8 6400^3: 32 % slower split), and pays
        // only when the tiles leave at least 7/8 of the resident workgroup
        // slots idle and every tile has a long K loop to share out (INT8
        // 256 x 256 x 65536: 2.1x faster split; 1024 x 1024 x 16384, 256
        // tiles of 128 stages: 6 % slower).
        if (T * 8 > G || KT < 128)
            return pl;
    }
    // The last full wave joins the stream-K part, so every workgroup runs
    // between 1 and 2 tiles of iterations there ("two-tile" hybrid).
    const int64_t tiles_dp = full >= 1 ? (full - 1) * G : 0;
    const int64_t sk_tiles = T - tiles_dp;
    const int64_t iters = sk_tiles * KT;
    const int64_t grid = iters < G ? iters : G;
    const int64_t need = 2 * grid * (int64_t)c.BM * c.BN * 4;
    if (need > partial_bytes || need > INT32_MAX || sk_tiles > flag_count || tiles_dp > INT32_MAX)
        return pl;
    pl.grid = (int)grid;
    pl.tiles_dp = (int)tiles_dp;
    pl.sk_tiles = (int)sk_tiles;
    pl.iters = iters;
    return pl;
}

template <int P>
static hipError_t launch_generic(const GemmProblem &p, hipStream_t stream);

template <int P, int BM, int BN, int BKB, int WGM, int WGN, int NS, int VAR = VAR_BASE>
static hipError_t launch_one(const GemmProblem &p, const StreamKPlan &sk, const TileWorkspace &ws,
                             hipStream_t stream) {
    if (p.kbytes < BKB)   // no full K tile: the ring kernel needs at least one
        return launch_generic<P>(p, stream);
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    dim3 block(64 * WGM * WGN);
    if (sk.grid > 0) {
        // the plan was made for this tile shape and workspace
        const bool dp_only = sk.sk_tiles == 0 && sk.iters == 0;   // persistent, every tile whole
        if (sk.tiles_dp + sk.sk_tiles != tiles_m * tiles_n || sk.sk_tiles > ws.flag_count ||
            (!dp_only && (2 * (int64_t)sk.grid * BM * BN * 4 > ws.partial_bytes || sk.iters < sk.grid)) ||
            sk.iters != (int64_t)sk.sk_tiles * ((p.kbytes + BKB - 1) / BKB))
            return hipErrorInvalidValue;
        StreamKArgs a;
        a.tiles_dp = sk.tiles_dp;
        a.iters = sk.iters;
        a.partial = ws.partial;
        a.partial_bytes = (int)(2 * (int64_t)sk.grid * BM * BN * 4);
        a.flags = ws.flags;
        hipLaunchKernelGGL((gemm_tile_sk_kernel<P, BM, BN, BKB, WGM, WGN, NS, VAR>), dim3(sk.grid), block,
                           0, stream, p, tiles_m, tiles_n, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_tile_kernel<P, BM, BN, BKB, WGM, WGN, NS, VAR>), dim3(tiles_m * tiles_n),
                       block, 0, stream, p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_pp(const GemmProblem &p, hipStream_t stream) {
    const int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    hipLaunchKernelGGL((gemm_pp_kernel<P>), dim3(tiles_m * tiles_n), dim3(512), 0, stream, p, tiles_m,
                       tiles_n);
    return hipGetLastError();
}

// B-direct kernel: data-parallel launches with K a whole number of stages;
// anything else goes to the ring kernel of the same tile shape.
template <int P, int NS>
static hipError_t launch_dtv(const GemmProblem &p, const StreamKPlan &sk, const TileWorkspace &ws,
                             hipStream_t stream) {
    if (sk.grid > 0 || p.kbytes % 128 != 0 || p.kbytes < 128)
        return launch_one<P, 256, 256, 128, 2, 2, 2>(p, sk, ws, stream);
    const int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    hipLaunchKernelGGL((gemm_dtv_kernel<P, NS>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, p,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_generic(const GemmProblem &p, hipStream_t stream) {
    constexpr int BM = 128, BN = 128;
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_tile_generic_kernel<P, BM, BN, 64, 2, 2>), dim3(tiles_m * tiles_n),
                       dim3(256), 0, stream, p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_prec(int cfg, const GemmProblem &p, const StreamKPlan &sk,
                              const TileWorkspace &ws, bool aligned, hipStream_t stream) {
    if (!aligned)   // byte-gather loads, one shape
        return launch_generic<P>(p, stream);
    switch (cfg) {
    case CFG_256x256: return launch_one<P, 256, 256, 64, 2, 2, 4>(p, sk, ws, stream);
    case CFG_128x128: return launch_one<P, 128, 128, 64, 2, 2, 4>(p, sk, ws, stream);
    case CFG_64x64: return launch_one<P, 64, 64, 128, 2, 2, 3>(p, sk, ws, stream);
    case CFG_256x128: return launch_one<P, 256, 128, 128, 2, 2, 3>(p, sk, ws, stream);
    case CFG_256x256_BK128: return launch_one<P, 256, 256, 128, 2, 2, 2>(p, sk, ws, stream);
    case CFG_128x256: return launch_one<P, 128, 256, 128, 2, 2, 3>(p, sk, ws, stream);
    case CFG_128x128_BK128: return launch_one<P, 128, 128, 128, 2, 2, 4>(p, sk, ws, stream);
    case CFG_256x256_W8: return launch_one<P, 256, 256, 128, 4, 2, 2>(p, sk, ws, stream);
    case CFG_256x256_W8_BK64: return launch_one<P, 256, 256, 64, 4, 2, 4>(p, sk, ws, stream);
    case CFG_256x128_2B: return launch_one<P, 256, 128, 64, 2, 2, 3>(p, sk, ws, stream);
    case CFG_128x128_2B: return launch_one<P, 128, 128, 128, 2, 2, 2>(p, sk, ws, stream);
    case CFG_128x256_2B: return launch_one<P, 128, 256, 64, 2, 2, 3>(p, sk, ws, stream);
    case CFG_256x256_PP:
        if constexpr (P != PREC_W4A4) {
            if (sk.grid == 0 && p.kbytes % 128 == 0 && p.kbytes >= 256)
                return launch_pp<P>(p, stream);
        }
        // stream-K, a partial K tile or the W4A4 epilogue: the ring kernel of
        // the same tile shape
        return launch_one<P, 256, 256, 128, 2, 2, 2>(p, sk, ws, stream);
    case CFG_256x256_SPLIT: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_SPLIT>(p, sk, ws, stream);
    case CFG_256x256_NT: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_NT>(p, sk, ws, stream);
    case CFG_256x256_SC1: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_SC1>(p, sk, ws, stream);
    case CFG_256x256_VGPR: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_VGPR>(p, sk, ws, stream);
    case CFG_256x256_SPREAD: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_SPREAD>(p, sk, ws, stream);
    case CFG_256x256_DTV: return launch_dtv<P, 2>(p, sk, ws, stream);
    case CFG_256x256_SC0: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_SC0>(p, sk, ws, stream);
    case CFG_256x256_EARLY: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_EARLY>(p, sk, ws, stream);
    case CFG_256x256_WEAVE: return launch_one<P, 256, 256, 128, 2, 2, 2, VAR_WEAVE>(p, sk, ws, stream);
    case CFG_64x64_DEEP: return launch_one<P, 64, 64, 128, 2, 2, 8>(p, sk, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_kn(int prec, const GemmProblem &p, hipStream_t stream) {
    const int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    const dim3 grid(tiles_m * tiles_n), block(256);
    switch (prec) {
    case PREC_F16: hipLaunchKernelGGL(gemm_tile_kn_kernel<PREC_F16>, grid, block, 0, stream, p, tiles_m, tiles_n); break;
    case PREC_I8: hipLaunchKernelGGL(gemm_tile_kn_kernel<PREC_I8>, grid, block, 0, stream, p, tiles_m, tiles_n); break;
    case PREC_I4: hipLaunchKernelGGL(gemm_tile_kn_kernel<PREC_I4>, grid, block, 0, stream, p, tiles_m, tiles_n); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int prec, int cfg, const GemmProblem &p, const StreamKPlan &sk,
                       const TileWorkspace &ws, hipStream_t stream) {
    // The fast kernel needs 16-byte aligned rows and 32-bit offsets within the
    // 256 rows of a tile.
    const int64_t kRowLimit = (int64_t)1 << 23;
    const bool aligned = (reinterpret_cast<uintptr_t>(p.A) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(p.B) % 16 == 0) && p.lda_b % 16 == 0 &&
                         p.ldb_b % 16 == 0 && p.lda_b < kRowLimit && p.ldb_b < kRowLimit;
    switch (prec) {
    case PREC_F16: return launch_prec<PREC_F16>(cfg, p, sk, ws, aligned, stream);
    case PREC_I8: return launch_prec<PREC_I8>(cfg, p, sk, ws, aligned, stream);
    case PREC_I4: return launch_prec<PREC_I4>(cfg, p, sk, ws, aligned, stream);
    case PREC_W4A4: return launch_prec<PREC_W4A4>(cfg, p, sk, ws, aligned, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mpg
