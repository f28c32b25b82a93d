// Weight-only INT4 GEMM Y = X * dequant(Wq)^T on gfx950 (fp16 activations,
// packed signed INT4 weights, per-(row, K-group) fp16 scales, fp16 output).
//
// Method ("fused-int4-gemm-sm75" README, project description and feature
// list): read packed INT4 weights straight from global memory, dequantise them
// in registers with no shared-memory round trip, multiply on the matrix unit,
// group_size = 128 scales. The README pads M to 16 so that every lane of the
// matrix instruction holds valid data; here lanes whose activation row is past
// M hold explicit zeros and their results are never stored.
//
// Layout of one step (128 consecutive k of 16 weight rows, one wavefront):
// lane l owns weight row n0 + l%16 and the 32-k run starting at
// 32 * (l/16); it loads those 16 packed bytes with one dwordx4. Each 8-nibble
// word becomes 8 fp16 values with an exact bit trick:
//   u = nibble ^ 8 = q + 8,  half(0x6400 | u) = 1024 + u,  minus 1032 -> q
// done for two nibbles at a time (nibbles j and j+4 of the word share one
// 32-bit register). The activations are loaded in the same k order, so four
// v_mfma_f32_16x16x32_f16 cover the 128 k of the step.
//
// Scales: when G is a multiple of 128 a step lies inside one group, the four
// MFMAs sum x*q exactly in fp32 and the group scale multiplies that sum
// (fp32). Otherwise the scale multiplies the fp16 weights before the MFMA.
#include "mpgemm_internal.h"
#include "lds_dma.h"

#include <algorithm>
#include <type_traits>
#include <climits>

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 8 packed nibbles (k = 0..7, low nibble first) -> 8 fp16 values of q in the
// order k = 0,4,1,5,2,6,3,7.
__device__ __forceinline__ f16x8 dequant8(uint32_t w) {
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t magic = 0x64006400u;
    uint32_t h0 = (u & 0x000F000Fu) | magic;
    uint32_t h1 = ((u >> 4) & 0x000F000Fu) | magic;
    uint32_t h2 = ((u >> 8) & 0x000F000Fu) | magic;
    uint32_t h3 = ((u >> 12) & 0x000F000Fu) | magic;
    const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    f16x2 q0 = __builtin_bit_cast(f16x2, h0) + bias;
    f16x2 q1 = __builtin_bit_cast(f16x2, h1) + bias;
    f16x2 q2 = __builtin_bit_cast(f16x2, h2) + bias;
    f16x2 q3 = __builtin_bit_cast(f16x2, h3) + bias;
    f16x8 r = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
    return r;
}

// 8 consecutive fp16 activations -> the order k = 0,4,1,5,2,6,3,7.
__device__ __forceinline__ f16x8 perm8(f16x8 x) {
    return __builtin_shufflevector(x, x, 0, 4, 1, 5, 2, 6, 3, 7);
}

// Loads and MFMAs of UU consecutive 128-k steps starting at step s0 for one
// wavefront (16 weight rows, MT blocks of 16 activation rows). Every load is
// issued before any is consumed, from clamped (always valid) addresses, so
// the loads stay in flight together; rows past M or N only feed results that
// are never stored. With KFULL false, lane groups whose 32-k run lies past K
// zero their weights and activations at use time.
template <int MT, int UU, bool SCALE_AFTER, bool KFULL>
__device__ __forceinline__ void w4a16_steps(const W4A16Problem &p, int s0, int lane, int nrow_c,
                                            int m0, int lg, f32x4 (&acc)[MT]) {
    const int g = lane >> 4;
    const uint8_t *wrow = p.W + (int64_t)nrow_c * p.ldw_b;
    const uint16_t *srow = p.S + (int64_t)nrow_c * p.lds;
    i32x4 wv[UU];
    _Float16 sc[UU];
    f16x8 xv[UU][MT][4];
    bool k_ok[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        int kl = (s0 + u) * 128 + g * 32;
        k_ok[u] = KFULL || kl < p.K;
        kl = (KFULL || kl < p.K) ? kl : p.K - 32;
        wv[u] = *reinterpret_cast<const i32x4 *>(wrow + kl / 2);
        sc[u] = __builtin_bit_cast(_Float16, srow[kl >> lg]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int mrow = m0 + mt * 16 + (lane & 15);
            mrow = mrow < p.M ? mrow : p.M - 1;
            const f16x8 *xp = reinterpret_cast<const f16x8 *>(p.X + (int64_t)mrow * p.ldx + kl);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xv[u][mt][t] = xp[t];
        }
    }
    // keep the scheduler from interleaving the load phase with the math
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        if constexpr (!KFULL) {
            if (!k_ok[u]) {
                wv[u] = i32x4{0, 0, 0, 0};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        xv[u][mt][t] = f16x8{};
            }
        }
        f16x8 wq[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            wq[t] = dequant8((uint32_t)wv[u][t]);
            if constexpr (!SCALE_AFTER) {
                const f16x8 s8 = {sc[u], sc[u], sc[u], sc[u], sc[u], sc[u], sc[u], sc[u]};
                wq[t] = wq[t] * s8;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (SCALE_AFTER) {
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(perm8(xv[u][mt][t]), wq[t], part, 0, 0, 0);
                const float sf = (float)sc[u];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[mt][r] += part[r] * sf;
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(perm8(xv[u][mt][t]), wq[t], acc[mt], 0, 0, 0);
            }
        }
    }
}

// MT: 16-row activation blocks per wavefront; WN: wavefronts along N (16 weight
// rows each); WK: wavefronts splitting K (reduced through LDS at the end);
// U: steps whose loads are issued before any of them is consumed.
template <int MT, int WN, int WK, int U, bool SCALE_AFTER, bool KFULL>
__global__ __launch_bounds__(64 * WN * WK) void w4a16_kernel(W4A16Problem p, int lg) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WN, wk = wave / WN;
    const int n0 = blockIdx.x * (16 * WN) + wn * 16;
    const int m0 = blockIdx.y * (16 * MT);
    const int nrow = n0 + (lane & 15);
    const int nrow_c = nrow < p.N ? nrow : p.N - 1;
    const int g = lane >> 4;

    const int steps = (p.K + 127) / 128;
    const int per_wave = (steps + WK - 1) / WK;
    const int s_begin = wk * per_wave;
    const int s_end = min(steps, s_begin + per_wave);

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    int s0 = s_begin;
    for (; s0 + U <= s_end; s0 += U)
        w4a16_steps<MT, U, SCALE_AFTER, KFULL>(p, s0, lane, nrow_c, m0, lg, acc);
    for (; s0 < s_end; ++s0)
        w4a16_steps<MT, 1, SCALE_AFTER, KFULL>(p, s0, lane, nrow_c, m0, lg, acc);

    // Reduce the WK partial sums (16x16 accumulator layout: register r of
    // lane l holds row 4*(l/16) + r, column l%16).
    if constexpr (WK > 1) {
        __shared__ f32x4 red[WK][WN][MT][64];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            red[wk][wn][mt][lane] = acc[mt];
        __syncthreads();
        if (wk != 0)
            return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            for (int o = 1; o < WK; ++o)
                acc[mt] += red[o][wn][mt][lane];
    }
    if (nrow >= p.N)
        return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + mt * 16 + 4 * g + r;
            if (m < p.M)
                p.Y[(int64_t)m * p.ldy + nrow] = __builtin_bit_cast(uint16_t, (_Float16)acc[mt][r]);
        }
}

// ---------------------------------------------------------------- GEMV path
//
// Decode shapes (a handful of activation rows) are a single pass over the
// weights. The MFMA layout above gives every lane its own activation row, so
// with M = 1 fifteen of every sixteen lanes load and multiply padding; here
// each lane instead owns a 32-k chunk of the K axis, keeps the activations of
// that chunk in registers, and reuses them for R weight rows. Products run on
// the VALU as fp16 pairs accumulated in fp32 (v_dot2_f32_f16).
//
// Dequantisation without a subtraction per weight: with u = nibble ^ 8 = q + 8,
// a 32-bit word of 8 nibbles (k = 0..7) gives four fp16 pairs by one mask-or
// each, two of them after one shift:
//   (u & 0x000F000F) | 0x64006400  -> (1024 + u_k0, 1024 + u_k4)
//   (u & 0x00F000F0) | 0x54005400  -> (  64 + u_k1,   64 + u_k5)
//   same on u >> 8                 -> k2, k6 (offset 1024) and k3, k7 (offset 64)
// (0x6400 is 1024 with a unit step; 0x5400 is 64 with a step of 1/16, so a
// nibble in mantissa bits 4..7 adds exactly u). The chunk's dot product
// therefore equals sum x*q + 1032 * (sum of x over k = 0, 2, 4, 6 mod 8) +
// 72 * (sum over k = 1, 3, 5, 7 mod 8); that correction depends on x only and
// is computed once per activation chunk. All products are exact in fp32.

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// Activation chunk (32 fp16, k order) -> pairs (k, k+4) of each 8-k word,
// in the order the weight pairs are produced: one byte permute per pair
// (v_perm_b32: selector bytes 0-3 pick the second source, 4-7 the first).
__device__ __forceinline__ void pair_x(const i32x4 (&xv)[4], uint32_t (&xp)[16]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t d0 = (uint32_t)xv[t][0], d1 = (uint32_t)xv[t][1];
        const uint32_t d2 = (uint32_t)xv[t][2], d3 = (uint32_t)xv[t][3];
        xp[4 * t + 0] = __builtin_amdgcn_perm(d2, d0, 0x05040100u);   // k0, k4
        xp[4 * t + 1] = __builtin_amdgcn_perm(d2, d0, 0x07060302u);   // k1, k5
        xp[4 * t + 2] = __builtin_amdgcn_perm(d3, d1, 0x05040100u);   // k2, k6
        xp[4 * t + 3] = __builtin_amdgcn_perm(d3, d1, 0x07060302u);   // k3, k7
    }
}

__device__ __forceinline__ float offset_of_chunk(const uint32_t (&xp)[16]) {
    const uint32_t c1032 = 0x64086408u;   // (1032, 1032)
    const uint32_t c72 = 0x54805480u;     // (72, 72)
    float a[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float &c = a[t & 1];
        c = dot2(xp[4 * t + 0], c1032, c);
        c = dot2(xp[4 * t + 1], c72, c);
        c = dot2(xp[4 * t + 2], c1032, c);
        c = dot2(xp[4 * t + 3], c72, c);
    }
    return a[0] + a[1];
}

// Masks and exponent patterns of the mask-or steps, held in VGPRs: gfx9's
// three-operand encoding takes no literal constant, so with literals each
// mask-or would split into an AND and an OR.
struct NibbleConsts {
    uint32_t m_lo, m_hi, e_lo, e_hi;
};

__device__ __forceinline__ NibbleConsts nibble_consts() {
    NibbleConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
    asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.e_lo), "+v"(k.e_hi));
    return k;
}

__device__ __forceinline__ float dot_chunk(const i32x4 w, const uint32_t (&xp)[16], const NibbleConsts &k) {
    float a[2] = {0.f, 0.f};   // two independent chains
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t u = (uint32_t)w[t] ^ 0x88888888u;
        const uint32_t hi = u >> 8;
        float &c = a[t & 1];
        c = dot2((u & k.m_lo) | k.e_lo, xp[4 * t + 0], c);
        c = dot2((u & k.m_hi) | k.e_hi, xp[4 * t + 1], c);
        c = dot2((hi & k.m_lo) | k.e_lo, xp[4 * t + 2], c);
        c = dot2((hi & k.m_hi) | k.e_hi, xp[4 * t + 3], c);
    }
    return a[0] + a[1];
}

// Sum over each row of 16 lanes with DPP moves (VALU latency, no LDS round
// trip): swap neighbours, swap pairs, then rotate the row by 4 and by 8.
// Every lane ends with the total of its 16-lane row.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));  // row_ror 4
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));  // row_ror 8
    return v;
}

// R: weight rows per wavefront; KS: wavefronts splitting K (4 / KS row groups
// per workgroup of 4 wavefronts); MM: activation rows per workgroup.
template <int R, int KS, int MM>
__global__ __launch_bounds__(256) void w4a16_gemv_kernel(W4A16Problem p, int lg) {
    constexpr int RG = 4 / KS;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kp = wave % KS, rg = wave / KS;
    const int n0 = (blockIdx.x * RG + rg) * R;
    const int m0 = blockIdx.y * MM;
    const int CK = p.K >> 5;
    const int cpk = (CK + KS - 1) / KS;
    const int c_begin = kp * cpk;
    const int c_end = min(CK, c_begin + cpk);

    const uint8_t *wrow[R];
    const uint16_t *srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = min(n0 + r, p.N - 1);
        wrow[r] = p.W + (int64_t)n * p.ldw_b;
        srow[r] = p.S + (int64_t)n * p.lds;
    }
    const uint16_t *xrow[MM];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm)
        xrow[mm] = p.X + (int64_t)min(m0 + mm, p.M - 1) * p.ldx;

    float acc[MM][R];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm)
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[mm][r] = 0.f;

    const NibbleConsts nk = nibble_consts();
    for (int c = c_begin + lane; c < c_end; c += 64) {
        // activations first, then scales and weight rows: the pairing and
        // the offset term (activations only) and the first rows' products
        // run while the later loads are still in flight
        i32x4 wv[R];
        uint16_t sv[R];
        i32x4 xv[MM][4];
#pragma unroll
        for (int mm = 0; mm < MM; ++mm)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xv[mm][t] = reinterpret_cast<const i32x4 *>(xrow[mm] + 32u * (uint32_t)c)[t];
#pragma unroll
        for (int r = 0; r < R; ++r)
            sv[r] = srow[r][(uint32_t)(32 * c) >> lg];
#pragma unroll
        for (int r = 0; r < R; ++r)
            wv[r] = *reinterpret_cast<const i32x4 *>(wrow[r] + 16u * (uint32_t)c);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < MM; ++mm) {
            uint32_t xp[16];
            pair_x(xv[mm], xp);
            const float off = offset_of_chunk(xp);
            // (scheduling fences: each row's products wait only for its own
            // weight load, not for the last one)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float s = (float)__builtin_bit_cast(_Float16, sv[r]);
                acc[mm][r] += (dot_chunk(wv[r], xp, nk) - off) * s;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Each wavefront leaves one partial per 16-lane row; one thread per output
    // adds the 4 * KS partials of its row.
    __shared__ float red[4][MM][R][4];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float t = row16_sum(acc[mm][r]);
            if ((lane & 15) == 0)
                red[wave][mm][r][lane >> 4] = t;
        }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < RG * MM * R) {
        const int g = t / (MM * R), mm = (t / R) % MM, r = t % R;
        float y = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                y += red[g * KS + k][mm][r][q];
        const int n = (blockIdx.x * RG + g) * R + r, m = m0 + mm;
        if (n < p.N && m < p.M)
            p.Y[(int64_t)m * p.ldy + n] = __builtin_bit_cast(uint16_t, (_Float16)y);
    }
}

// ---------------------------------------------------------------- MFMA GEMV path
//
// Decode shapes on the matrix unit. The VALU GEMV above spends most of its
// instructions on the dot products; here v_mfma_f32_16x16x32_f16 takes them
// and the VALU only dequantises, with the mask-or scheme of the GEMV (6
// operations per 8 weights, pairs (k, k+4), values offset + u). A workgroup
// owns 16 weight rows (the MFMA's columns) and all of K. Its MM activation
// rows are the MFMA's rows 0 .. MM-1 (the other rows repeat the last one and
// are never stored); they are staged once into LDS, already in the pair
// order of the weights, and the staging pass also computes, per row and
// 128-k step, the offset term c = sum over the step of 1032 x_k (k = 0..3
// mod 8 in the low halves of the pairs of slots 0 and 2) and 72 x_k (slots 1
// and 3). Each step's first MFMA starts from -c instead of 0, so the step ends
// at sum x q exactly as in the GEMV, and one FMA applies the group scale (G a
// multiple of 128: a step lies in one group).
//
// The NW wavefronts split K into contiguous step ranges. Lane (n, j) =
// (lane % 16, lane / 16) loads the 16-byte run of 32 k at 32 j of each 128-k
// step of weight row n; its word t (k = 32 j + 8 t ... + 7) is the B operand
// of the step's MFMA t, and lane (m, j) reads the matching activations of row
// m from LDS (all 16 lanes of a lane group read one address: a broadcast).
// All weight loads of SPW steps are issued before the staging arithmetic.
// The NW partial results meet in LDS and are added in wavefront order.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int NW, int MM, int SPW, int XPR>
__global__ __launch_bounds__(NW * 64) void w4a16_gemv_mfma_kernel(W4A16Problem p, int lg) {
    extern __shared__ __align__(16) uint8_t gm_smem[];
    constexpr int NT = NW * 64;
    const int K = p.K, S = K >> 7, CPR = K >> 3;   // 128-k steps, 16-byte chunks per row
    uint16_t *xs = reinterpret_cast<uint16_t *>(gm_smem);                         // MM x K, pair order
    float *negc = reinterpret_cast<float *>(gm_smem + (size_t)MM * K * 2);        // [S][MM]
    float *red = negc + (size_t)S * MM;                                            // [NW][MM][16]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 16, m0 = blockIdx.y * MM;
    const int nl = lane & 15, j = lane >> 4;

    // 1. this thread's activation chunks (chunk c = tid + u NT of each row)
    i32x4 xr[MM][XPR];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
        const uint16_t *xrow = p.X + (int64_t)min(m0 + mm, p.M - 1) * p.ldx;
#pragma unroll
        for (int u = 0; u < XPR; ++u) {
            // unconditional (clamped) loads keep the code straight, so the
            // wait for them leaves the weight loads below in flight
            const int c = min(tid + u * NT, CPR - 1);
            xr[mm][u] = *reinterpret_cast<const i32x4 *>(xrow + 8 * c);
        }
    }

    // 2. the weight runs and scales of the first SPW steps of this wavefront
    const int spw = (S + NW - 1) / NW;
    const int s_begin = min(S, wave * spw), s_end = min(S, s_begin + spw);
    const int nrow = min(n0 + nl, p.N - 1);
    const uint8_t *wrow = p.W + (int64_t)nrow * p.ldw_b + 16 * j;
    const uint16_t *srow = p.S + (int64_t)nrow * p.lds;
    i32x4 wv[SPW];
    uint16_t sv[SPW];
    auto issue = [&](int c0) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            // a step past the range reloads the last one of the matrix (a
            // wavefront with no steps at all loads it too, and uses nothing)
            const int sg = c0 + i < s_end ? c0 + i : S - 1;
            wv[i] = *reinterpret_cast<const i32x4 *>(wrow + 64u * (uint32_t)sg);
            sv[i] = srow[(uint32_t)(128 * sg) >> lg];
        }
    };
    issue(s_begin);
    __builtin_amdgcn_sched_barrier(0);

    // 3. pair the activations, store them, and the negated offset term of
    //    every (row, step): the 16 chunks of a step sit in one 16-lane row
    const uint32_t c1032 = 0x64086408u, c72 = 0x54805480u;
#pragma unroll
    for (int mm = 0; mm < MM; ++mm)
#pragma unroll
        for (int u = 0; u < XPR; ++u) {
            const int c = tid + u * NT;
            if (c < CPR) {   // uniform over each 16-lane row (CPR is a multiple of 16)
                const i32x4 v = xr[mm][u];
                const uint32_t d0 = (uint32_t)v[0], d1 = (uint32_t)v[1], d2 = (uint32_t)v[2], d3 = (uint32_t)v[3];
                u32x4 pr;
                pr[0] = __builtin_amdgcn_perm(d2, d0, 0x05040100u);   // k0, k4
                pr[1] = __builtin_amdgcn_perm(d2, d0, 0x07060302u);   // k1, k5
                pr[2] = __builtin_amdgcn_perm(d3, d1, 0x05040100u);   // k2, k6
                pr[3] = __builtin_amdgcn_perm(d3, d1, 0x07060302u);   // k3, k7
                float a0 = dot2(pr[0], c1032, 0.f), a1 = dot2(pr[1], c72, 0.f);
                a0 = dot2(pr[2], c1032, a0);
                a1 = dot2(pr[3], c72, a1);
                const float t = row16_sum(a0 + a1);
                *reinterpret_cast<u32x4 *>(xs + (size_t)mm * K + 8 * c) = pr;
                if ((lane & 15) == 0)
                    negc[(c >> 4) * MM + mm] = -t;
            }
        }
    __syncthreads();

    // 4. the steps: MFMA t of a step takes word t of every lane's run
    const NibbleConsts nk = nibble_consts();
    float y[MM];
#pragma unroll
    for (int r = 0; r < MM; ++r)
        y[r] = 0.f;
    const uint16_t *xa = xs + (size_t)min(nl, MM - 1) * K + 32 * j;
    for (int c0 = s_begin; c0 < s_end; c0 += SPW) {
        if (c0 != s_begin)
            issue(c0);
        // two steps at a time on independent accumulators (the 4 MFMAs of a
        // step form one dependent chain); the second of an odd last pair
        // repeats the first and is not added
        static_assert(SPW % 2 == 0, "steps in pairs");
#pragma unroll
        for (int i = 0; i < SPW; i += 2) {
            const int sg0 = c0 + i;
            if (sg0 >= s_end)
                break;
            const bool has1 = sg0 + 1 < s_end;
            const int sg[2] = {sg0, has1 ? sg0 + 1 : sg0};
            f32x4 acc[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (MM == 4) {
                    acc[h] = *reinterpret_cast<const f32x4 *>(negc + 4 * sg[h]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[h][r] = negc[sg[h] * MM + min(r, MM - 1)];
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(xa + 128 * sg[h] + 8 * t);
                    const uint32_t u = (uint32_t)wv[i + h][t] ^ 0x88888888u;
                    const uint32_t hi = u >> 8;
                    u32x4 b;
                    b[0] = (u & nk.m_lo) | nk.e_lo;
                    b[1] = (u & nk.m_hi) | nk.e_hi;
                    b[2] = (hi & nk.m_lo) | nk.e_lo;
                    b[3] = (hi & nk.m_hi) | nk.e_hi;
                    acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, b), acc[h], 0, 0, 0);
                }
            const float sc0 = (float)__builtin_bit_cast(_Float16, sv[i]);
            const float sc1 = has1 ? (float)__builtin_bit_cast(_Float16, sv[i + 1]) : 0.f;
#pragma unroll
            for (int r = 0; r < MM; ++r)
                y[r] = __builtin_fmaf(sc1, acc[1][r], __builtin_fmaf(sc0, acc[0][r], y[r]));
        }
    }

    // 5. rows 0 .. MM-1 are registers 0 .. MM-1 of lanes 0-15; add the NW
    //    wavefronts' results in order
    if (j == 0) {
#pragma unroll
        for (int r = 0; r < MM; ++r)
            red[(wave * MM + r) * 16 + nl] = y[r];
    }
    __syncthreads();
    if (tid < MM * 16) {
        const int r = tid >> 4, n = tid & 15;
        float v = red[r * 16 + n];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            v += red[(w * MM + r) * 16 + n];
        if (m0 + r < p.M && n0 + n < p.N)
            p.Y[(int64_t)(m0 + r) * p.ldy + n0 + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
}

// ---------------------------------------------------------------- slice MFMA path
//
// Mid-size and prefill M. The weights dominate the bytes and the activations
// are reused by every output column, so a workgroup keeps the activations of
// its K range (BM rows) in LDS (resident, or streamed through a few slots),
// loaded with direct-to-LDS loads in the conflict-free layout described at
// the kernel. Its wavefronts stream their weight rows straight into
// registers, a fixed number of 128-k steps ahead of the products, dequantise
// them exactly, multiply by the group scale in fp16 and feed
// v_mfma_f32_16x16x32_f16 (the fused-int4-gemm-sm75 README dequantises to
// fp16 in registers before the matrix product).
//
// Dequantisation in natural k order, so the activations need no reordering
// (dequant8_perm below): with u = nibble ^ 8 = q + 8, the fp16 patterns 0x6400
// (1024, unit step) and 0x5400 (64, step 1/16) around nibbles 2b and 2b+1 give
// the pair (1024 + u_2b, 64 + u_2b+1), and subtracting (1032, 72) gives q
// exactly.
//
// The 4 wavefronts are arranged WN (columns) x WK (K quarters); the WK
// partial sums meet in LDS. When the grid still has too few workgroups, K is
// also split over KS workgroups: each writes its fp32 partial tile to the
// workspace and a second kernel adds the slices in slice order.

// 8 packed nibbles (k = 0..7, low nibble first) -> 8 fp16 values q * s in
// natural k order, 16 VALU operations: per byte b, one byte permute of the
// word and a constant builds (byte, 0x64, byte, 0x54), one three-input bit
// operation keeps the even-k nibble in bits 0-3 and the odd-k one in bits
// 4-7 of the two bytes while flipping their top bits (u = nibble ^ 8 = q + 8),
// so the halves read 1024 + u and 64 + u'; subtracting (1032, 72) leaves q
// exactly, and one multiply applies the scale. The three constants sit in
// VGPRs (gfx9's three-operand encoding takes no literal).
struct PermConsts {
    uint32_t expo, mask, flip;
};

__device__ __forceinline__ PermConsts perm_consts() {
    PermConsts k{0x00005464u, 0xFFF0FF0Fu, 0x00800008u};
    asm volatile("" : "+v"(k.expo), "+v"(k.mask), "+v"(k.flip));
    return k;
}

__device__ __forceinline__ f16x8 dequant8_perm(uint32_t w, f16x2 s2, const PermConsts &k) {
    const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-72.0f};
    f16x2 q[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // result bytes: w.b, expo.0, w.b, expo.1 (v_perm: selector 0-3 pick the
        // second source's bytes, 4-7 the first's)
        const uint32_t sel = (uint32_t)b | (4u << 8) | ((uint32_t)b << 16) | (5u << 24);
        const uint32_t pr = (__builtin_amdgcn_perm(k.expo, w, sel) & k.mask) ^ k.flip;
        q[b] = (__builtin_bit_cast(f16x2, pr) + bias) * s2;
    }
    return f16x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
}

// Consecutive workgroup ids go round-robin over the 8 XCDs; renumber them so
// that each XCD gets a contiguous range of logical ids (neighbouring K slices
// and tiles then share that XCD's L2).
__device__ __forceinline__ int xcd_contiguous(int id, int nblk) {
    if (nblk < 8)
        return id;
    const int xcd = id % 8, local = id / 8;
    const int base = nblk / 8, rem = nblk % 8;
    return xcd * base + (xcd < rem ? xcd : rem) + local;
}


// KF: K is a multiple of 128 (so are the K slices), every step that starts
// inside the range lies wholly inside it, and the load clamps are scalar.
template <int MB, int NB, int WN, int WK, int NST, int PDT, int RG, bool KF>
__global__ __launch_bounds__(256) void w4a16_slice_kernel(W4A16Problem p, W4A16Split sk, int lg) {
    static_assert(WN * WK == 4, "4 wavefronts");
    constexpr int BM = 16 * MB, BN = 16 * NB * WN;
    // LDS: the workgroup's NST * WK blocks of 128 k, block-major. Block b
    // holds two halves of 64 k (BM rows of 128 bytes each); row r's 16-byte
    // chunk c of a half sits at slot c ^ ((r / 2) & 7). MFMA lane group g
    // takes the 32-k quarter pi(g) = 0, 2, 1, 3 (g = 0..3) of each 128 k, for
    // the weights and the activations alike, so that lanes l and l + 16 read
    // the same slot of the same row in the two halves (BM * 128 bytes apart,
    // the same 16-byte bank group), and lanes 0-15 read 16 rows at 16
    // distinct bank groups: the fragment reads are free of bank conflicts. A
    // direct-to-LDS unit (1 KiB) is 8 whole rows of one half: every 128-byte
    // line of X is fetched once.
    constexpr int PB = BM * 128, BLOCK = 2 * PB;   // bytes per half, per block
    constexpr int NBLK = NST * WK;
    constexpr int XU = WK * MB;                  // direct-to-LDS loads per wavefront per step
    constexpr int WL = 2 * NB;                   // weight + scale loads per wavefront per step
    constexpr int PD = PDT < NST ? PDT : NST;    // steps of loads in flight ahead of the products
    static_assert((PD - 1) * (XU + WL) < 64 && NST * WL < 64, "vmcnt of the step waits");
    // RG > 0: the blocks stream through RG LDS slots (block b in slot b % RG)
    // instead of all staying resident; the loads of step s + PD go out after
    // the barrier of step s, when every wavefront is done with step s - 1, so
    // RG = PD + 1 slots suffice
    static_assert(RG == 0 || (WK == 1 && PD < NST && RG >= PD + 1), "activation ring");
    constexpr int NSLOT = RG > 0 ? RG : NBLK;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    // explicitly uniform: the direct-to-LDS destinations derived from it
    // then live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wk = wave / WN;

    // Workgroup -> (column group, row block, K slice). Consecutive workgroup
    // ids go round-robin over the 8 XCDs; give each XCD a contiguous range so
    // the K slices and row blocks of one column group share an L2.
    const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
    const int ks = logical % sk.ks;
    const int tile = logical / sk.ks;          // = ng * mblocks + mb
    const int mb = tile % sk.mblocks, ng = tile / sk.mblocks;
    const int m0 = mb * BM;
    const int k_begin = ks * sk.kslice;
    const int k_end = min(p.K, k_begin + sk.kslice);
    const int kw = k_begin + wk * 128 * NST;    // this wavefront's K range starts here
    const int n0w = ng * BN + wn * 16 * NB;
    __shared__ __attribute__((aligned(16))) uint8_t xs[NSLOT * BLOCK];

    const uint8_t *wrow[NB];
    const uint16_t *srow[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int n = min(n0w + 16 * j + (lane & 15), p.N - 1);
        wrow[j] = p.W + (int64_t)n * p.ldw_b;
        srow[j] = p.S + (int64_t)n * p.lds;
    }
    // lane l of an activation unit (8 rows of one half) covers row
    // 8 q + l / 8 and chunk c = (l % 8) ^ ((row / 2) % 8) of its slot l % 8
    const int pig = ((g & 1) << 1) | (g >> 1);   // this lane group's quarter
    const uint16_t *xrow[XU];
    int xc8[XU];
#pragma unroll
    for (int v = 0; v < XU; ++v) {
        const int q = (wave + 4 * v) % (2 * MB);
        const int r = 8 * q + (lane >> 3);
        xrow[v] = p.X + (int64_t)min(m0 + r, p.M - 1) * p.ldx;
        xc8[v] = 8 * ((lane & 7) ^ ((r >> 1) & 7));
    }
    i32x4 wr[NST][NB];
    uint16_t sr[NST][NB];
    // Loads of step s: block wk' * NST + s of every wavefront group wk'
    // (activations, direct to LDS, shared by the workgroup) and this
    // wavefront's weights and scales of its block s. Clamped addresses: rows
    // past M and k past the range only meet zero weights or outputs that are
    // never stored.
    auto issue_x = [&](int s) {
#pragma unroll
        for (int v = 0; v < XU; ++v) {
            const int u = wave + 4 * v;                 // unit of this step: (block group, half, rows)
            const int b = (u / (4 * MB)) * NST + s;     // block
            const int h = (u / (2 * MB)) % 2, q = u % (2 * MB);   // half, 8-row group
            int k;
            if constexpr (KF)
                k = min(k_begin + 128 * b, p.K - 128) + 64 * h + xc8[v];   // scalar clamp
            else
                k = min(k_begin + 128 * b + 64 * h + xc8[v], p.K - 8);
            dma16(xrow[v] + k, xs + (RG > 0 ? b % RG : b) * BLOCK + h * PB + q * 1024);
        }
        asm volatile("" ::: "memory");
    };
    auto issue_w = [&](int s) {
        int k;
        if constexpr (KF) {
            k = min(kw + 128 * s, p.K - 128) + 32 * pig;   // scalar clamp
        } else {
            k = kw + 128 * s + 32 * pig;
            k = k + 32 <= p.K ? k : p.K - 32;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            wr[s][j] = *reinterpret_cast<const i32x4 *>(wrow[j] + (k >> 1));
            sr[s][j] = srow[j][k >> lg];
        }
        asm volatile("" ::: "memory");
    };
    // PD < NST: step by step (activations, then weights, of each step);
    // PD = NST: every activation load first, then the weights, so that the
    // products can start once the activations alone have landed
#pragma unroll
    for (int s = 0; s < PD; ++s) {
        issue_x(s);
        if constexpr (PD < NST)
            issue_w(s);
    }
    if constexpr (PD == NST) {
#pragma unroll
        for (int s = 0; s < NST; ++s)
            issue_w(s);
    }

    // products step by step; each step first waits for its own loads (the
    // younger ones are the next steps', at most PD - 1 of them), then puts
    // the loads of step s + PD in flight
    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const PermConsts pk = perm_consts();
    // per-lane part of the fragment address of MFMA step t: quarter pi(g)
    // (half pi(g) / 2, chunks 4 (pi(g) % 2) + t), row 16 i + l % 16 (16 i
    // does not change the swizzle bits)
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = lane & 15;
        aoff[t] = (pig >> 1) * PB + r * 128 + (((4 * (pig & 1) + t) ^ ((r >> 1) & 7)) * 16);
    }
#pragma unroll
    for (int s = 0; s < NST; ++s) {
        if (PD < NST || s == 0) {
            // with every step issued up front (PD = NST) one wait covers all
            // activations: the younger loads are all the weights
            const int younger = (s + PD <= NST ? PD : NST - s) - 1;
            wait_vm_lds_n(PD < NST ? younger * (XU + WL) : NST * WL);
            lds_barrier();
        }
        if (s + PD < NST) {
            issue_x(s + PD);
            issue_w(s + PD);
        }
        if (kw + 128 * s >= k_end)
            continue;   // (the barriers above stay uniform across the wavefronts)
        const bool live = KF || kw + 128 * s + 32 * pig < k_end;
        const uint8_t *blk = xs + (RG > 0 ? (wk * NST + s) % RG : wk * NST + s) * BLOCK;
        // every fragment of the step in its own registers: all LDS reads go
        // out at once and the dequantisation runs in their shadow, then the
        // MFMAs follow back to back (with one set of fragment registers
        // reused per k-step, each k-step waited on its reads and on the
        // previous MFMAs' operand reads before its dequantisation)
        f16x8 a[4][MB];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < MB; ++i)
                a[t][i] = *reinterpret_cast<const f16x8 *>(blk + aoff[t] + i * 2048);
        f16x8 b[4][NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const _Float16 sc = __builtin_bit_cast(_Float16, sr[s][j]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // a run past the K range gets q = 0 (u = 8 in every nibble)
                const uint32_t w = live ? (uint32_t)wr[s][j][t] : 0u;
                b[t][j] = dequant8_perm(w, f16x2{sc, sc}, pk);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][i], b[t][j], acc[i][j], 0, 0, 0);
    }

    // 4. add the WK partial sums through LDS (reusing the activation buffer)
    if constexpr (WK > 1) {
        static_assert(NSLOT * BLOCK >= 4 * MB * NB * 4 * 64 * 4, "reduction buffer");
        __syncthreads();
        f32x4 *red = reinterpret_cast<f32x4 *>(xs);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                red[((wave * MB + i) * NB + j) * 64 + lane] = acc[i][j];
        __syncthreads();
        if (wk != 0)
            return;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int o = 1; o < WK; ++o)
                    acc[i][j] += red[(((o * WN + wn) * MB + i) * NB + j) * 64 + lane];
    }

    // 5. store Y directly, or this K slice's fp32 partial tile in the
    //    threads' own register order (every store instruction writes 1 KiB
    //    of contiguous memory); w4a16_reduce_kernel maps it back to (m, n)
    if (sk.ks == 1) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 16 * i + 4 * g + r, n = n0w + 16 * j + (lane & 15);
                    if (m < p.M && n < p.N)
                        p.Y[(int64_t)m * p.ldy + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][r]);
                }
        return;
    }
    // only the wavefronts with wk == 0 get here; they are the first WN
    float *mine = sk.partial + (int64_t)logical * (BM * BN);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mine[((i * NB + j) * 4 + r) * (64 * WN) + tid] = acc[i][j][r];
}

// ---------------------------------------------------------------- producer/consumer slices
//
// The slice kernel's wavefronts both issue their loads and run the products,
// and a load that the memory system cannot take yet holds up the wavefront's
// instruction stream, MFMAs included: with the weights cold, a wavefront of
// the 64 x 128 slices spends about a third of its time in load issue (clock
// stamps per wavefront). Here the roles are split: the last 4 wavefronts
// only move the activations and the weights of each 128-k step into an
// R-slot LDS ring with direct-to-LDS loads, keeping up to R - 1 steps in
// flight, and the first NC only read LDS, dequantise and run the MFMAs (the
// tile and partial layout of the slice kernel with NC column wavefronts, so
// its K-slice sum kernel applies). One barrier per step: before barrier s the
// producers have waited for step s's loads and the consumers have finished
// step s - 1, whose slot the producers refill with step s + R - 1 after it.
//
// Slot layout: the activation block of the slice kernel (two 64-k halves of
// BM rows x 128 bytes, chunk c of row r at c ^ ((r / 2) & 7)), then the
// weights, tile row n's 64 bytes at 64 n with its 16-byte quarter q at slot
// q ^ ((n / 4) & 3) (one direct-to-LDS load moves 16 whole rows; the slots
// make the 16 rows a consumer lane group reads hit 16 bank groups). The
// group scales of the workgroup's whole K range sit in a table filled by the
// consumers before the first barrier. K must be a multiple of 128.
template <int MB, int NB, int NC, int R, int NSTMAX>
__global__ __launch_bounds__((NC + 4) * 64) void w4a16_pc_kernel(W4A16Problem p, W4A16Split sk, int lg) {
    constexpr int WN = NC, BM = 16 * MB, BN = 16 * NB * WN, CT = NC * 64;
    constexpr int PB = BM * 128, XBLK = 2 * PB, WBLK = BN * 64, SLOT = XBLK + WBLK;
    constexpr int XUP = XBLK / 1024 / 4, WUP = WBLK / 1024 / 4;   // loads per producer per step
    static_assert(XUP == MB && WUP * 4 * 16 == BN, "units");
    __shared__ __attribute__((aligned(16))) uint8_t ring[R * SLOT];
    __shared__ uint16_t stab[NSTMAX * 4 * BN];   // [step][quarter][column]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
    const int ks = logical % sk.ks;
    const int tile = logical / sk.ks;
    const int mb = tile % sk.mblocks, ng = tile / sk.mblocks;
    const int m0 = mb * BM, n0 = ng * BN;
    const int k_begin = ks * sk.kslice;
    const int k_end = min(p.K, k_begin + sk.kslice);
    const int NS = (k_end - k_begin) >> 7;   // steps of this workgroup (K % 128 == 0)

    if (wave >= NC) {
        // ------------------------------------------------ producers
        const int pw = wave - NC;
        // activation unit u = pw + 4 v (half u / (2 MB), 8-row group u % (2 MB));
        // lane l: row 8 q + l / 8, chunk (l % 8) ^ ((row / 2) % 8)
        const uint16_t *xsrc[XUP];
        int xdst[XUP];
#pragma unroll
        for (int v = 0; v < XUP; ++v) {
            const int u = pw + 4 * v;
            const int h = u / (2 * MB), q = u % (2 * MB);
            const int r = 8 * q + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            xsrc[v] = p.X + (int64_t)min(m0 + r, p.M - 1) * p.ldx + k_begin + 64 * h + 8 * c;
            xdst[v] = h * PB + q * 1024;
        }
        // weight unit wu = pw + 4 v: tile rows 16 wu ... + 15, lane l: row
        // 16 wu + l / 4, slot l % 4 holding quarter (l % 4) ^ ((row / 4) & 3)
        const uint8_t *wsrc[WUP];
#pragma unroll
        for (int v = 0; v < WUP; ++v) {
            const int wu = pw + 4 * v;
            const int row = 16 * wu + (lane >> 2);
            const int q = (lane & 3) ^ ((row >> 2) & 3);
            wsrc[v] = p.W + (int64_t)min(n0 + row, p.N - 1) * p.ldw_b + (k_begin >> 1) + 16 * q;
        }
        auto issue = [&](int s) {
            uint8_t *slot = ring + (s % R) * SLOT;
#pragma unroll
            for (int v = 0; v < XUP; ++v)
                dma16(xsrc[v] + 128 * s, slot + xdst[v]);
#pragma unroll
            for (int v = 0; v < WUP; ++v)
                dma16(wsrc[v] + 64 * s, slot + XBLK + (pw + 4 * v) * 1024);
            asm volatile("" ::: "memory");
        };
        for (int s = 0; s < R - 1 && s < NS; ++s)
            issue(s);
        for (int s = 0; s < NS; ++s) {
            // outstanding: steps s ... min(s + R - 2, NS - 1); step s must have landed
            const int younger = min(R - 2, NS - 1 - s);
            wait_vm_lds_n(younger * (XUP + WUP));
            lds_barrier();
            if (s + R - 1 < NS)
                issue(s + R - 1);
        }
        return;
    }

    // ---------------------------------------------------- consumers
    const int wn = wave, g = lane >> 4;
    const int pig = ((g & 1) << 1) | (g >> 1);   // this lane group's 32-k quarter
    const int n0w = n0 + wn * 16 * NB;
    // the scale table: entry (s, q, col) = S[n0 + col][(k_begin + 128 s + 32 q) >> lg]
    for (int e = tid; e < NS * 4 * BN; e += CT) {
        const int col = e % BN, q = (e / BN) % 4, st = e / (4 * BN);
        const int n = min(n0 + col, p.N - 1);
        stab[e] = p.S[(int64_t)n * p.lds + ((k_begin + 128 * st + 32 * q) >> lg)];
    }
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = lane & 15;
        aoff[t] = (pig >> 1) * PB + r * 128 + (((4 * (pig & 1) + t) ^ ((r >> 1) & 7)) * 16);
    }
    int woff[NB], soff[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int row = wn * 16 * NB + 16 * j + (lane & 15);
        woff[j] = XBLK + row * 64 + ((pig ^ ((row >> 2) & 3)) * 16);
        soff[j] = pig * BN + row;
    }
    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const PermConsts pk = perm_consts();
    for (int s = 0; s < NS; ++s) {
        wait_lds_only();   // the scale table (s = 0) and this wavefront's reads of step s - 1
        lds_barrier();
        const uint8_t *slot = ring + (s % R) * SLOT;
        i32x4 wv[NB];
        _Float16 sc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            wv[j] = *reinterpret_cast<const i32x4 *>(slot + woff[j]);
            sc[j] = __builtin_bit_cast(_Float16, stab[s * 4 * BN + soff[j]]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f16x8 a[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                a[i] = *reinterpret_cast<const f16x8 *>(slot + aoff[t] + i * 2048);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const f16x8 b = dequant8_perm((uint32_t)wv[j][t], f16x2{sc[j], sc[j]}, pk);
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b, acc[i][j], 0, 0, 0);
            }
        }
    }

    // store Y directly, or this K slice's partial tile in the slice kernel's
    // register order (consumer thread tid = 64 wn + lane)
    if (sk.ks == 1) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 16 * i + 4 * g + r, n = n0w + 16 * j + (lane & 15);
                    if (m < p.M && n < p.N)
                        p.Y[(int64_t)m * p.ldy + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][r]);
                }
        return;
    }
    float *mine = sk.partial + (int64_t)logical * (BM * BN);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mine[((i * NB + j) * 4 + r) * (64 * WN) + tid] = acc[i][j][r];
}

// Y = fp16(sum of the KS fp32 partial tiles), slices added in slice order.
// Partial tile layout (as written by w4a16_slice_kernel): element
// ((i * NB + j) * 4 + r) * (64 * WN) + t holds row 16 i + 4 ((t % 64) / 16) + r
// and column (t / 64) * 16 NB + 16 j + t % 16 of the BM x BN tile. Four
// consecutive elements (t % 4 == 0) are four consecutive columns of one row:
// one thread adds them as a 16-byte vector per slice and stores 4 fp16.
template <int MB, int NB, int WN>
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(W4A16Problem p, W4A16Split sk) {
    constexpr int BM = 16 * MB, BN = 16 * NB * WN, TILE = BM * BN;
    static_assert(TILE % 4 == 0 && (64 * WN) % 4 == 0, "vector groups");
    // the same XCD-contiguous renumbering as the slice kernel, so that the
    // workgroups adding a tile's slices run on the XCD whose L2 wrote them
    const int64_t e = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
    const int64_t tiles = (int64_t)sk.mblocks * sk.ngroups;
    if (e >= tiles * (TILE / 4))
        return;
    const int tile = (int)(e / (TILE / 4)), q = 4 * (int)(e % (TILE / 4));
    const int t = q % (64 * WN), reg = q / (64 * WN);
    const int r = reg % 4, j = (reg / 4) % NB, i = reg / (4 * NB);
    const int lane = t % 64, wn = t / 64;
    const int mb = tile % sk.mblocks, ng = tile / sk.mblocks;
    const int m = mb * BM + 16 * i + 4 * (lane / 16) + r;
    const int n = ng * BN + wn * 16 * NB + 16 * j + lane % 16;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(sk.partial + (int64_t)tile * sk.ks * TILE + q);
    f32x4 y = src[0];
    for (int o = 1; o < sk.ks; ++o)
        y += src[(int64_t)o * (TILE / 4)];
    if (m >= p.M)
        return;
    uint16_t *dst = p.Y + (int64_t)m * p.ldy + n;
    if (n + 4 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<f16x4 *>(dst) = f16x4{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (n + c < p.N)
                dst[c] = __builtin_bit_cast(uint16_t, (_Float16)y[c]);
    }
}

// ---------------------------------------------------------------------------
// Larger M: w4a16_ring_kernel. One 128 x 64 output tile per workgroup. The
// activations stream through a ring of LDS stages (128 rows x 128 k, 32 KiB)
// next to the tile's packed weights (64 rows x 128 k, 4 KiB), both moved by
// direct-to-LDS loads. Within a stage each of the 4 wavefronts takes 32 k for
// all 128 rows, so every dequantised weight word feeds 4 MFMAs
// (v_mfma_f32_32x32x16_f16); the 4 partial tiles meet in LDS at the end.
// When the tiles alone would leave compute units idle, K is also split over
// KS workgroups: each writes an fp32 slice of Y (row-major, padded to whole
// tiles) and w4a16_rowsum_kernel adds the slices in slice order.
//
// k order inside a wavefront's 32 k (four runs of 8): at MFMA step t (0, 1)
// lane half h = l / 32 supplies run 2h + t of both operands, so a lane gets
// its two weight words of a column with one 8-byte LDS read.
//
// LDS layouts (16-byte chunks): activation row r holds its 16 chunks with
// chunk c at slot c ^ (r & 15); weight row n holds 4 chunks (32 k each) with
// chunk c at slot c ^ ((n / 4) & 3). Fragment reads are then free of bank
// conflicts, and the direct-to-LDS loads, which write lane-contiguous 16-byte
// slots, fetch the permuted global chunk instead.
constexpr int RG_BM = 128, RG_BN = 64, RG_BK = 128;
constexpr int RG_XST = RG_BM * RG_BK * 2;            // activation bytes per stage
constexpr int RG_WST = RG_BN * RG_BK / 2;            // packed weight bytes per stage
constexpr int RG_STAGE = RG_XST + RG_WST;
constexpr int RG_RED = 4 * 32 * 64 * 16;             // the 4 wavefronts' fp32 tiles
constexpr int RG_PER = RG_XST / (256 * 16) + 1;      // direct-to-LDS loads per thread per stage

// LDS of one workgroup: NSTG ring slots, then a table of fp16 scales (spr
// entries per weight row, what is left of the 160 KiB). The epilogue's 4
// partial tiles (32 KiB each) reuse the ring and, with 3 stages, the table.
template <int NSTG>
struct RingLds {
    static constexpr int spr = NSTG == 3 ? 384 : 128;
    static constexpr int ring = NSTG * RG_STAGE;
    static constexpr int bytes = ring + RG_BN * spr * 2;
    static_assert(bytes <= 160 * 1024 && bytes >= RG_RED, "LDS");
};
static int ring_spr(int cfg) { return cfg == W4A16_RING3_128x64 ? RingLds<3>::spr : RingLds<4>::spr; }

// A 16-byte direct-to-LDS load (lane l writes lds + 16 l) issued through
// inline assembly, so the compiler neither counts it nor waits for it before
// LDS reads: every consumer waits with wait_vm_lds<> and a barrier. (The
// compiler's own tracking of such loads cannot tell ring slots apart and
// would wait for all of them before any read.)
// M0 (the LDS base of the load) is saved and restored around it.
__device__ __forceinline__ void dma16_untracked(const void *g, const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(base)
                 : "memory");
}
// The same with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (global_load_lds_dwordx4 v_off, s_base): no per-lane address
// arithmetic when only the base moves.
__device__ __forceinline__ void dma16_untracked_sb(uint32_t voff, const void *sbase, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory");
}
// A 2-byte global load into a VGPR, untracked likewise: its value may be used
// only after a wait that covers it and untracked_ready().
__device__ __forceinline__ uint32_t load_u16_untracked(const uint16_t *g) {
    uint32_t v;
    asm volatile("global_load_ushort %0, %1, off" : "=v"(v) : "v"(g) : "memory");
    return v;
}
__device__ __forceinline__ void untracked_ready(uint32_t &v) { asm volatile("" : "+v"(v)); }

// s_waitcnt for "at most `ahead` stages of direct-to-LDS loads still in
// flight" (0 <= ahead <= NSTG).
template <int NSTG>
__device__ __forceinline__ void ring_wait(int ahead) {
    if constexpr (NSTG >= 4) {
        if (ahead >= 4) {
            wait_vm_lds<4 * RG_PER>();
            return;
        }
    }
    if (ahead >= 3)
        wait_vm_lds<3 * RG_PER>();
    else if (ahead == 2)
        wait_vm_lds<2 * RG_PER>();
    else if (ahead == 1)
        wait_vm_lds<RG_PER>();
    else
        wait_vm_lds<0>();
}

// One wavefront's operands of one stage: activation fragments a[t][i] and
// packed weight words with their scales (before dequantisation), and the
// dequantised weight fragments b[t][j].
struct RingRaw {
    f16x8 a[2][4];
    uint32_t wq[2][2];
    f16x2 sc[2];   // the group scale in both halves
};
struct RingFrag {
    f16x8 a[2][4];
    f16x8 b[2][2];
};

template <int NSTG>
__global__ __launch_bounds__(256) void w4a16_ring_kernel(W4A16Problem p, W4A16Split sk, int lg) {
    static_assert(NSTG == 3 || NSTG == 4, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t smem[RingLds<NSTG>::bytes];
    uint16_t *tab = reinterpret_cast<uint16_t *>(smem + RingLds<NSTG>::ring);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
    const int ks = logical % sk.ks, tile = logical / sk.ks;
    const int mb = tile % sk.mblocks, ng = tile / sk.mblocks;
    const int m0 = mb * RG_BM, n0 = ng * RG_BN;
    const int k_begin = ks * sk.kslice;
    const int k_end = min(p.K, k_begin + sk.kslice);
    const int nst = (k_end - k_begin + RG_BK - 1) / RG_BK;    // stages (the last may be partial)
    const int nfull = (k_end - k_begin) / RG_BK;               // whole stages
    auto kstage = [&](int t) { return k_begin + t * RG_BK; };   // first k of stage t

    // scale table tab[(g - g0) * 64 + n] (group-major: the lanes of a read
    // take consecutive columns), first pass (up to 64 groups: 16 per
    // thread), loaded ahead of the ring so that it lands with stage 0
    const int g0 = k_begin >> lg;
    const int gcnt = ((k_end - 1) >> lg) - g0 + 1;
    const int wcol = tid >> 2;
    const uint16_t *srow = p.S + (int64_t)min(n0 + wcol, p.N - 1) * p.lds + g0;
    uint32_t sv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
        sv[e] = load_u16_untracked(srow + min((tid & 3) + 4 * e, gcnt - 1));

    // direct-to-LDS sources: 8 activation chunks (4 rows per wavefront
    // instruction) and 1 weight chunk per thread and stage. Rows past M or N
    // are clamped (their results are never stored); k is clamped to K (runs
    // past the slice are zeroed before use).
    const int xk = 8 * ((lane & 15) ^ ((4 * wave + (lane >> 4)) & 15));
    const uint16_t *xrow[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = 4 * (wave + 4 * v) + (lane >> 4);
        xrow[v] = p.X + (int64_t)min(m0 + r, p.M - 1) * p.ldx;
    }
    const int wk = 32 * ((tid & 3) ^ ((wcol >> 2) & 3));
    const uint8_t *wrow = p.W + (int64_t)min(n0 + wcol, p.N - 1) * p.ldw_b;
    // whole stages (k0 + 128 <= K): uniform bases plus per-lane byte offsets
    // that stay fixed (the host keeps 128 ldx * 2 and 64 ldw_b below 2^32)
    uint32_t xoff[8];
#pragma unroll
    for (int v = 0; v < 8; ++v)
        xoff[v] = (uint32_t)((xrow[v] - p.X - (int64_t)m0 * p.ldx + xk) * 2);
    const uint32_t woff = (uint32_t)((wrow - p.W) - (int64_t)n0 * p.ldw_b + (wk >> 1));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)smem;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int q, int s) {   // stage s into ring slot q
        const int k0 = kstage(s);
        const uint32_t lslot = lds0 + q * RG_STAGE + wave_u * 1024;
        if (k0 + RG_BK <= p.K) {
            const uint16_t *xb = p.X + (int64_t)m0 * p.ldx + k0;
            const uint8_t *wb = p.W + (int64_t)n0 * p.ldw_b + (k0 >> 1);
#pragma unroll
            for (int v = 0; v < 8; ++v)
                dma16_untracked_sb(xoff[v], xb, lslot + 4 * v * 1024);
            dma16_untracked_sb(woff, wb, lslot + RG_XST);
        } else {
            const uint8_t *base = smem + q * RG_STAGE;
            const int kx = min(k0 + xk, p.K - 8);
#pragma unroll
            for (int v = 0; v < 8; ++v)
                dma16_untracked(xrow[v] + kx, base + (wave + 4 * v) * 1024);
            dma16_untracked(wrow + (min(k0 + wk, p.K - 32) >> 1), base + RG_XST + wave * 1024);
        }
    };
    // fill the whole ring: stage s + NSTG later goes into the slot of stage s
    // once every wavefront has read stage s. All NSTG slots are loaded even
    // when the slice has fewer stages (copies of its last stage, never read):
    // with no branch between the untracked scale loads above and their use
    // below, the compiler cannot merge their registers with early copies.
#pragma unroll
    for (int q = 0; q < NSTG; ++q)
        issue(q, min(q, nst - 1));

    // stage 0 (and, being older, the scale loads) landed
    wait_vm_lds<(NSTG - 1) * RG_PER>();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        untracked_ready(sv[e]);
        const int g = (tid & 3) + 4 * e;
        if (g < gcnt)
            tab[g * RG_BN + wcol] = (uint16_t)sv[e];
    }
    // more than 64 groups: further passes (their loads are tracked, so the
    // compiler waits for them, and with them for the ring)
    for (int e0 = 64; e0 < gcnt; e0 += 64) {
        uint16_t v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            v[e] = srow[min(e0 + (tid & 3) + 4 * e, gcnt - 1)];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int g = e0 + (tid & 3) + 4 * e;
            if (g < gcnt)
                tab[g * RG_BN + wcol] = v[e];
        }
        wait_vm_lds<0>();   // no tracked load left in flight past this point
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    const int xa = (lane & 31) * 256;     // this lane's activation row within a 32-row block
    // LDS reads of this wavefront's 32 k of stage s (in ring slot q); with
    // TAIL, runs past the slice read as zeros
    auto read_raw = [&](int q, int s, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        const uint8_t *base = smem + q * RG_STAGE;
        const int kw = kstage(s) + 32 * wave;
        const bool live = !TAIL || kw < k_end;
        RingRaw R;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 32 * j + (lane & 31);
            const uint64_t d = *reinterpret_cast<const uint64_t *>(
                base + RG_XST + col * 64 + 16 * (wave ^ ((col >> 2) & 3)) + 8 * h);
            R.wq[j][0] = live ? (uint32_t)d : 0u;
            R.wq[j][1] = live ? (uint32_t)(d >> 32) : 0u;
            const _Float16 sc = __builtin_bit_cast(_Float16, tab[(((live ? kw : k_begin) >> lg) - g0) * RG_BN + col]);
            R.sc[j] = f16x2{sc, sc};
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int xc = 16 * ((4 * wave + 2 * h + t) ^ (lane & 15));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                R.a[t][i] = *reinterpret_cast<const f16x8 *>(base + i * 32 * 256 + xa + xc);
                if constexpr (TAIL)
                    R.a[t][i] = live ? R.a[t][i] : f16x8{};
            }
        }
        return R;
    };
    const PermConsts pk = perm_consts();
    auto dequant = [&](const RingRaw &R, RingFrag &F) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                F.a[t][i] = R.a[t][i];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                F.b[t][j] = dequant8_perm(R.wq[j][t], R.sc[j], pk);
        }
    };
    auto mfma = [&](const RingFrag &F) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[t][i], F.b[t][j], acc[i][j], 0, 0, 0);
    };

    RingFrag F0, F1;
    lds_barrier();   // stage 0 and the scale table visible
    if (0 < nfull)
        dequant(read_raw(0, 0, std::false_type{}), F0);
    else
        dequant(read_raw(0, 0, std::true_type{}), F0);

    // One step (stage s in `cur`, in ring slot q): wait until stage s + 1 has
    // landed and publish it (the barrier also certifies that every wavefront
    // has read stage s), refill slot q with stage s + NSTG, read stage s + 1,
    // then the MFMAs of stage s with the dequantisation of stage s + 1 in
    // their shadow. The steady form runs only where the refill is real and
    // stage s + 1 whole, so exactly NSTG - 2 stages after s + 1 are in flight
    // at the wait; it has no branch (the accumulators stay in place).
    int q = 0;
    auto next_slot = [&](int x) { return x + 1 == NSTG ? 0 : x + 1; };
    // The 9 direct-to-LDS loads of the refill are spread over the 16 MFMAs
    // (one per MFMA pair, in explicit scheduling segments): issued together,
    // they queue in the compute unit's load path and stall the in-order
    // instruction stream with the matrix unit idle.
    auto step_steady = [&](int s, const RingFrag &cur, RingFrag &nxt) {
        wait_vm_lds<(NSTG - 2) * RG_PER>();
        lds_barrier();
        const int qn = next_slot(q);
        __builtin_amdgcn_sched_barrier(0);
        const RingRaw R = read_raw(qn, s + 1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        // the refill is a whole stage (the steady condition keeps it below nfull)
        const int k0 = kstage(s + NSTG);
        const uint32_t lslot = lds0 + q * RG_STAGE + wave_u * 1024;
        const uint16_t *xb = p.X + (int64_t)m0 * p.ldx + k0;
        const uint8_t *wb = p.W + (int64_t)n0 * p.ldw_b + (k0 >> 1);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            dma16_untracked_sb(xoff[g], xb, lslot + 4 * g * 1024);
            __builtin_amdgcn_sched_barrier(0);
            const int t = g / 4, j = (g / 2) % 2, i0 = 2 * (g % 2);
            acc[i0][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[t][i0], cur.b[t][j], acc[i0][j], 0, 0, 0);
            acc[i0 + 1][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[t][i0 + 1], cur.b[t][j], acc[i0 + 1][j], 0, 0, 0);
            if (g >= 4) {
                const int tt = (g - 4) / 2, jj = (g - 4) % 2;
                nxt.b[tt][jj] = dequant8_perm(R.wq[jj][tt], R.sc[jj], pk);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        dma16_untracked_sb(woff, wb, lslot + RG_XST);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                nxt.a[t][i] = R.a[t][i];
        q = qn;
    };
    int s = 0;
    for (; s + 1 + NSTG < nfull; s += 2) {
        step_steady(s, F0, F1);
        step_steady(s + 1, F1, F0);
    }
    // drain: at most NSTG + 2 stages remain, stage s in F0; after the last
    // stage the reads are of a stale slot and their result is unused
    auto step_drain = [&](int x, const RingFrag &cur, RingFrag &nxt) {
        ring_wait<NSTG>(max(0, min(NSTG - 2, nst - x - 2)));
        lds_barrier();
        if (x + NSTG < nst)
            issue(q, x + NSTG);
        q = next_slot(q);
        const RingRaw R = read_raw(q, x + 1, std::true_type{});
        mfma(cur);
        dequant(R, nxt);
    };
    if (s < nst)
        step_drain(s, F0, F1);
    if (s + 1 < nst)
        step_drain(s + 1, F1, F0);
    if (s + 2 < nst)
        step_drain(s + 2, F0, F1);
    if (s + 3 < nst)
        step_drain(s + 3, F1, F0);
    if (s + 4 < nst)
        step_drain(s + 4, F0, F1);
    if constexpr (NSTG == 4)
        if (s + 5 < nst)
            step_drain(s + 5, F1, F0);

    // the 4 partial tiles meet in LDS (every load has landed, the ring is
    // free): wavefront w leaves the row blocks of the other three in its
    // 32 KiB, wavefront v then adds the 4 partials of row block v in
    // wavefront order
    __syncthreads();
    f32x4 *red = reinterpret_cast<f32x4 *>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i != wave)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    red[(wave * 32 + (i * 2 + j) * 4 + qq) * 64 + lane] =
                        f32x4{acc[i][j][4 * qq], acc[i][j][4 * qq + 1], acc[i][j][4 * qq + 2], acc[i][j][4 * qq + 3]};
    __syncthreads();
    // 32x32 accumulator layout: register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int f = (wave * 2 + j) * 4 + qq;
            f32x4 own{};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i == wave)
                    own = f32x4{acc[i][j][4 * qq], acc[i][j][4 * qq + 1], acc[i][j][4 * qq + 2], acc[i][j][4 * qq + 3]};
            f32x4 y = wave == 0 ? own : red[f * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4; ++w)
                y += wave == w ? own : red[(w * 32 + f) * 64 + lane];
            const int ml = 32 * wave + 8 * qq + 4 * h;
            const int n = n0 + 32 * j + (lane & 31);
            if (sk.ks == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + ml + e;
                    if (m < p.M && n < p.N)
                        p.Y[(int64_t)m * p.ldy + n] = __builtin_bit_cast(uint16_t, (_Float16)y[e]);
                }
            } else {
                // tile-major slices: tile t's slice ks is one 128 x 64 block
                float *dst = sk.partial + (((int64_t)tile * sk.ks + ks) * RG_BM + ml) * RG_BN + (n - n0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[e * RG_BN] = y[e];
            }
        }
}

// Y = fp16(sum of the KS fp32 slices written by w4a16_ring_kernel), slices
// added in slice order; one thread per 4 consecutive columns of a tile row,
// 8 workgroups per 128 x 64 tile. Workgroups are renumbered like the ring
// kernel's, so the ones adding a tile run on the XCD whose L2 holds its
// slices.
__global__ __launch_bounds__(256) void w4a16_rowsum_kernel(W4A16Problem p, W4A16Split sk) {
    constexpr int TPT = RG_BM * RG_BN / 4;   // threads per tile
    const int64_t e = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
    const int tile = (int)(e / TPT), q = (int)(e % TPT);
    if (tile >= sk.mblocks * sk.ngroups)
        return;
    const int ml = q / (RG_BN / 4), nl = 4 * (q % (RG_BN / 4));
    const int m = (tile % sk.mblocks) * RG_BM + ml, n = (tile / sk.mblocks) * RG_BN + nl;
    if (m >= p.M || n >= p.N)
        return;
    const int64_t slice = (int64_t)RG_BM * RG_BN;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(sk.partial + (int64_t)tile * sk.ks * slice + ml * RG_BN + nl);
    f32x4 y = src[0];
    for (int o = 1; o < sk.ks; ++o)
        y += src[o * (slice / 4)];
    uint16_t *dst = p.Y + (int64_t)m * p.ldy + n;
    if (n + 4 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        const f16x4 o = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
        *reinterpret_cast<f16x4 *>(dst) = o;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (n + c < p.N)
                dst[c] = __builtin_bit_cast(uint16_t, (_Float16)y[c]);
    }
}


template <int MT, int WN, int WK, int U>
static hipError_t launch_cfg(const W4A16Problem &p, hipStream_t stream, int lg) {
    dim3 block(64 * WN * WK);
    dim3 grid((p.N + 16 * WN - 1) / (16 * WN), (p.M + 16 * MT - 1) / (16 * MT));
    // G % 128 == 0 implies K % 128 == 0: every step lies in one group
    if (p.G % 128 == 0)
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, true, true>), grid, block, 0, stream, p, lg);
    else if (p.K % 128 == 0)
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, false, true>), grid, block, 0, stream, p, lg);
    else
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, false, false>), grid, block, 0, stream, p, lg);
    return hipGetLastError();
}

template <int R, int KS, int MM>
static hipError_t launch_gemv_mm(const W4A16Problem &p, hipStream_t stream, int lg) {
    constexpr int rows_per_block = R * (4 / KS);
    dim3 grid((p.N + rows_per_block - 1) / rows_per_block, (p.M + MM - 1) / MM);
    hipLaunchKernelGGL((w4a16_gemv_kernel<R, KS, MM>), grid, dim3(256), 0, stream, p, lg);
    return hipGetLastError();
}

template <int R, int KS>
static hipError_t launch_gemv(const W4A16Problem &p, hipStream_t stream, int lg) {
    if (p.M == 1)
        return launch_gemv_mm<R, KS, 1>(p, stream, lg);
    if (p.M == 2)
        return launch_gemv_mm<R, KS, 2>(p, stream, lg);
    return launch_gemv_mm<R, KS, 4>(p, stream, lg);
}

// LDS of the MFMA GEMV: MM activation rows in pair order, the offset terms,
// the wavefront partials.
static constexpr int64_t GEMV_MFMA_LDS_MAX = 64 * 1024;
static int64_t gemv_mfma_lds(int mm, int nw, int64_t K) {
    return mm * K * 2 + (K / 128) * mm * 4 + (int64_t)nw * mm * 16 * 4;
}

// Steps whose loads a wavefront issues together: the whole range of a
// 4096-k row at the workgroup's wavefront count (a larger chunk would only
// reload the last step into the unused slots).
template <int NW, int MM, int XPR>
static hipError_t launch_gemv_mfma_mm(const W4A16Problem &p, hipStream_t stream, int lg) {
    constexpr int SPW = NW >= 16 ? 2 : (NW >= 8 ? 4 : 8);
    dim3 grid((p.N + 15) / 16, (p.M + MM - 1) / MM);
    const size_t lds = (size_t)gemv_mfma_lds(MM, NW, p.K);
    hipLaunchKernelGGL((w4a16_gemv_mfma_kernel<NW, MM, SPW, XPR>), grid, dim3(NW * 64), lds, stream, p, lg);
    return hipGetLastError();
}

// G a multiple of 128, the activation rows of a workgroup within 64 KiB of
// LDS and within what the threads stage in one pass (K <= 2048 XPR NW / 4);
// other shapes run the VALU GEMV.
template <int NW>
static hipError_t launch_gemv_mfma(const W4A16Problem &p, hipStream_t stream, int lg) {
    const int mm = p.M == 1 ? 1 : p.M == 2 ? 2 : 4;
    const int64_t chunks = p.K / 8;
    if (lg < 7 || gemv_mfma_lds(mm, NW, p.K) > GEMV_MFMA_LDS_MAX || chunks > 4 * NW * 64)
        return p.M == 1 ? launch_gemv<2, 2>(p, stream, lg) : launch_gemv<4, 2>(p, stream, lg);
    // activation chunks each thread stages: 1, 2 or 4
    const int xpr = chunks <= NW * 64 ? 1 : (chunks <= 2 * NW * 64 ? 2 : 4);
    auto go = [&](auto mmc) {
        constexpr int MMC = decltype(mmc)::value;
        return xpr == 1   ? launch_gemv_mfma_mm<NW, MMC, 1>(p, stream, lg)
               : xpr == 2 ? launch_gemv_mfma_mm<NW, MMC, 2>(p, stream, lg)
                          : launch_gemv_mfma_mm<NW, MMC, 4>(p, stream, lg);
    };
    if (mm == 1)
        return go(std::integral_constant<int, 1>{});
    if (mm == 2)
        return go(std::integral_constant<int, 2>{});
    return go(std::integral_constant<int, 4>{});
}

template <int MB, int NB, int WN, int WK, int NST, int PD, int RG>
static hipError_t launch_slice(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                               hipStream_t stream, int lg) {
    constexpr int BM = 16 * MB, BN = 16 * NB * WN;
    W4A16Split sk;
    sk.mblocks = plan.mblocks;
    sk.ngroups = plan.ngroups;
    sk.ks = plan.ks;
    sk.kslice = plan.kslice;
    sk.partial = ws.partial;
    const int64_t tiles = (int64_t)sk.mblocks * sk.ngroups;
    const int64_t blocks = tiles * sk.ks;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    if (p.K % 128 == 0)
        hipLaunchKernelGGL((w4a16_slice_kernel<MB, NB, WN, WK, NST, PD, RG, true>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, p, sk, lg);
    else
        hipLaunchKernelGGL((w4a16_slice_kernel<MB, NB, WN, WK, NST, PD, RG, false>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, p, sk, lg);
    if (sk.ks == 1)
        return hipGetLastError();
    const int64_t total = tiles * BM * BN / 4;   // one thread per 4 outputs
    hipLaunchKernelGGL((w4a16_reduce_kernel<MB, NB, WN>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, p, sk);
    return hipGetLastError();
}

// K % 128 != 0 runs the equivalent slice kernel (64 x 128, 8 steps).
template <int MB, int NB, int NC, int R, int NSTMAX>
static hipError_t launch_pc(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                            hipStream_t stream, int lg) {
    if (p.K % 128 != 0 || plan.kslice > 128 * NSTMAX)
        return launch_slice<MB, 2, 4, 1, NSTMAX, 2, 0>(p, plan, ws, stream, lg);
    static_assert(NB * NC == 8, "the fallback's 64 x 128 tile");
    constexpr int BM = 16 * MB, BN = 16 * NB * NC;
    W4A16Split sk;
    sk.mblocks = plan.mblocks;
    sk.ngroups = plan.ngroups;
    sk.ks = plan.ks;
    sk.kslice = plan.kslice;
    sk.partial = ws.partial;
    const int64_t tiles = (int64_t)sk.mblocks * sk.ngroups;
    const int64_t blocks = tiles * sk.ks;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((w4a16_pc_kernel<MB, NB, NC, R, NSTMAX>), dim3((unsigned)blocks), dim3((NC + 4) * 64), 0,
                       stream, p, sk, lg);
    if (sk.ks == 1)
        return hipGetLastError();
    const int64_t total = tiles * BM * BN / 4;
    hipLaunchKernelGGL((w4a16_reduce_kernel<MB, NB, NC>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       p, sk);
    return hipGetLastError();
}

template <int MT, int WN, int WK, int U>
static hipError_t launch_cfg(const W4A16Problem &p, hipStream_t stream, int lg);

template <int NSTG>
static hipError_t launch_ring(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                              hipStream_t stream, int lg) {
    // the ring kernel's per-lane load offsets are 32-bit: 128 activation rows
    // and 64 weight rows of the strides must span less than 4 GiB
    if (p.ldx * 2 * RG_BM >= ((int64_t)1 << 32) || p.ldw_b * RG_BN >= ((int64_t)1 << 32))
        return launch_cfg<2, 4, 1, 2>(p, stream, lg);
    W4A16Split sk;
    sk.mblocks = plan.mblocks;
    sk.ngroups = plan.ngroups;
    sk.ks = plan.ks;
    sk.kslice = plan.kslice;
    sk.partial = ws.partial;
    const int64_t blocks = (int64_t)sk.mblocks * sk.ngroups * sk.ks;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((w4a16_ring_kernel<NSTG>), dim3((unsigned)blocks), dim3(256), 0, stream, p, sk, lg);
    if (sk.ks == 1)
        return hipGetLastError();
    const int64_t threads = (int64_t)sk.mblocks * sk.ngroups * (RG_BM * RG_BN / 4);
    hipLaunchKernelGGL(w4a16_rowsum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p, sk);
    return hipGetLastError();
}

// The slice configurations: (configuration, MB, NB, WN, WK, NST). One list
// feeds both the host planning and the kernel dispatch.
// (config, MB, NB, WN, WK, NST, PD, RG): tile 16 MB x 16 NB WN, WK
// wavefronts along K, NST steps of 128 k per wavefront, loads PD steps
// ahead, activations resident (RG = 0) or through an RG-slot ring
#define MPG_SLICE_CONFIGS(X)                       \
    X(W4A16_SLICE_16x16_K4, 1, 1, 1, 4, 8, 8, 0)   \
    X(W4A16_SLICE_32x32_K2, 2, 1, 2, 2, 8, 2, 0)   \
    X(W4A16_SLICE_64x128, 4, 2, 4, 1, 8, 2, 0)     \
    X(W4A16_SLICE_128x128, 8, 2, 4, 1, 4, 2, 0)    \
    X(W4A16_SLICE_64x128_S4, 4, 2, 4, 1, 4, 2, 0)  \
    X(W4A16_SLICE_128x64_RING, 8, 1, 4, 1, 8, 2, 3)

// The producer/consumer slices, in the same shape notation (pd = ring slots).
#define MPG_PC_CONFIGS(X)                 \
    X(W4A16_PC_64x128, 4, 2, 4, 1, 8, 4, 0) \
    X(W4A16_PC_64x128_C8, 4, 1, 8, 1, 8, 4, 0)

W4A16Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int cfg, int cu_count, int64_t partial_floats) {
    W4A16Plan plan{K == 0 ? (int)W4A16_GEMV_R2_KS2 : cfg, 1, 0, 0, 0};
    int MB = 0, NB = 0, WN = 0, WK = 0, NST = 0;
    switch (plan.cfg) {
#define MPG_SHAPE(C, mb, nb, wn, wk, nst, pd, rg) \
    case C: MB = mb; NB = nb; WN = wn; WK = wk; NST = nst; break;
        MPG_SLICE_CONFIGS(MPG_SHAPE)
        MPG_PC_CONFIGS(MPG_SHAPE)
#undef MPG_SHAPE
    case W4A16_RING3_128x64:
    case W4A16_RING4_128x64: {
        plan.mblocks = (int)((M + RG_BM - 1) / RG_BM);
        plan.ngroups = (int)((N + RG_BN - 1) / RG_BN);
        const int64_t tiles = (int64_t)plan.mblocks * plan.ngroups;
        const int64_t steps = (K + RG_BK - 1) / RG_BK;
        int64_t ks = 1;
        while (tiles * ks < cu_count && ks < steps)
            ++ks;
        // equal slices in whole stages; a slice touches at most 4 spk + 1
        // groups (G >= 32), which the LDS scale table must hold
        int64_t spk = (steps + ks - 1) / ks;
        spk = std::min<int64_t>(spk, (ring_spr(plan.cfg) - 1) / 4);
        ks = (steps + spk - 1) / spk;
        if (ks > 1 && ks * plan.mblocks * RG_BM * plan.ngroups * RG_BN > partial_floats) {
            plan.cfg = W4A16_MFMA_TILE;
            plan.mblocks = plan.ngroups = 0;
            return plan;
        }
        plan.ks = (int)ks;
        plan.kslice = (int)(RG_BK * spk);
        return plan;
    }
    default: return plan;   // GEMV and the older MFMA kernels split K inside the workgroup
    }
    const int64_t BM = 16 * MB, BN = 16 * NB * WN, KSPAN = 128 * NST * WK;
    plan.mblocks = (int)((M + BM - 1) / BM);
    plan.ngroups = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)plan.mblocks * plan.ngroups;
    // K slices: at least K / KSPAN (what one workgroup holds), more while the
    // grid would leave compute units idle
    int64_t ks = (K + KSPAN - 1) / KSPAN;
    while (tiles * ks < cu_count && (ks + 1) * 128 <= K)
        ++ks;
    // equal slices in whole 128-k steps
    const int64_t steps = (K + 127) / 128;
    const int64_t spk = (steps + ks - 1) / ks;
    ks = (steps + spk - 1) / spk;
    if (ks > 1 && tiles * ks * BM * BN > partial_floats) {
        // the workspace cannot hold the partial tiles: a kernel that splits K
        // inside its workgroups instead
        plan.cfg = M <= 16 ? W4A16_MFMA_DECODE : W4A16_MFMA_TILE;
        plan.mblocks = plan.ngroups = 0;
        return plan;
    }
    plan.ks = (int)ks;
    plan.kslice = (int)(128 * spk);
    return plan;
}

int64_t w4a16_plan_scratch_floats(const W4A16Plan &plan) {
    if (plan.ks <= 1)
        return 0;
    switch (plan.cfg) {
#define MPG_SCRATCH(C, mb, nb, wn, wk, nst, pd, rg) \
    case C: return (int64_t)plan.ks * plan.mblocks * plan.ngroups * (16 * mb) * (16 * nb * wn);
        MPG_SLICE_CONFIGS(MPG_SCRATCH)
        MPG_PC_CONFIGS(MPG_SCRATCH)
#undef MPG_SCRATCH
    case W4A16_RING3_128x64:
    case W4A16_RING4_128x64:
        return (int64_t)plan.ks * plan.mblocks * RG_BM * plan.ngroups * RG_BN;
    default: return 0;
    }
}

const char *w4a16_cfg_name(int cfg) {
    static const char *names[W4A16_CFG_COUNT] = {
        "mfma 16 rows x 16 cols, K split 4", "mfma 32 x 64 tile",
        "gemv R1 KS2", "gemv R2 KS2", "gemv R4 KS2", "gemv R2 KS1", "gemv R4 KS1", "gemv R8 KS1",
        "slice 16 x 16, K over 4 wavefronts", "slice 32 x 32, K over 2 wavefronts",
        "slice 64 x 128", "slice 128 x 128", "ring 128 x 64, 3 stages", "ring 128 x 64, 4 stages",
        "slice 64 x 128, 4 stages (two workgroups per compute unit)",
        "slice 128 x 64, 8 stages through a 3-slot activation ring",
        "mfma gemv, 16 rows per workgroup, K over 4 wavefronts",
        "mfma gemv, 16 rows per workgroup, K over 8 wavefronts",
        "slice 64 x 128, 4 producer + 4 consumer wavefronts, 4-slot LDS ring",
        "slice 64 x 128, 4 producer + 8 consumer wavefronts, 4-slot LDS ring",
        "mfma gemv, 16 rows per workgroup, K over 16 wavefronts"};
    return cfg >= 0 && cfg < W4A16_CFG_COUNT ? names[cfg] : "?";
}

int choose_w4a16_cfg(int64_t M, int64_t N, int64_t K) {
    (void)N;
    (void)K;
    // measured at N = K = 4096 (cold weights, HIP graph replay): from 65 to
    // 128 rows the 64 x 128 slices win (M = 80: 12.6 vs 14.9 us for the ring
    // kernel, M = 128: 12.7 vs 15.0), above 128 the ring kernel (M = 160: 19.5
    // vs 20.4 us, 256: 20.0 vs 22.7; 512: 27.4 vs 45.0)
    // M = 1: the VALU GEMV (4.22 us against 4.49 for the matrix-unit GEMV,
    // whose one wavefront per SIMD with 8 weight loads each waits longer on
    // the cold weights than the GEMV's four with 2 each); 2 ... 4 rows: the
    // matrix-unit GEMV, whose arithmetic does not grow with M (M = 2: 4.56
    // vs 5.16 us, M = 4: 4.81 vs 6.70; VALU GEMV for G < 128)
    if (M == 1)
        return W4A16_GEMV_R2_KS2;
    if (M <= 4)
        return W4A16_GEMV_MFMA_NW4;
    if (M <= 16)
        return W4A16_SLICE_16x16_K4;
    if (M <= 32)
        return W4A16_SLICE_32x32_K2;
    // 33 ... 64 rows: the 64 x 128 slices over 4 stages of K, two workgroups
    // per compute unit (M = 48 and 64: 10.6 vs 13.4 us for the 32 x 32 slices)
    if (M <= 64)
        return W4A16_SLICE_64x128_S4;
    if (M <= 128)
        return W4A16_SLICE_64x128;
    return W4A16_RING3_128x64;
}

static hipError_t launch_one(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                             hipStream_t stream, int lg) {
    switch (plan.cfg) {
    case W4A16_MFMA_DECODE: return launch_cfg<1, 1, 4, 8>(p, stream, lg);
    case W4A16_MFMA_TILE: return launch_cfg<2, 4, 1, 2>(p, stream, lg);
    case W4A16_GEMV_R1_KS2: return launch_gemv<1, 2>(p, stream, lg);
    case W4A16_GEMV_R2_KS2: return launch_gemv<2, 2>(p, stream, lg);
    case W4A16_GEMV_R4_KS2: return launch_gemv<4, 2>(p, stream, lg);
    case W4A16_GEMV_R2_KS1: return launch_gemv<2, 1>(p, stream, lg);
    case W4A16_GEMV_R4_KS1: return launch_gemv<4, 1>(p, stream, lg);
    case W4A16_GEMV_R8_KS1: return launch_gemv<8, 1>(p, stream, lg);
    case W4A16_GEMV_MFMA_NW4: return launch_gemv_mfma<4>(p, stream, lg);
    case W4A16_GEMV_MFMA_NW8: return launch_gemv_mfma<8>(p, stream, lg);
    case W4A16_GEMV_MFMA_NW16: return launch_gemv_mfma<16>(p, stream, lg);
#define MPG_LAUNCH(C, mb, nb, wn, wk, nst, pd, rg) \
    case C: return launch_slice<mb, nb, wn, wk, nst, pd, rg>(p, plan, ws, stream, lg);
        MPG_SLICE_CONFIGS(MPG_LAUNCH)
#undef MPG_LAUNCH
#define MPG_LAUNCH_PC(C, mb, nb, wn, wk, nst, pd, rg) \
    case C: return launch_pc<mb, nb, wn, pd, nst>(p, plan, ws, stream, lg);
        MPG_PC_CONFIGS(MPG_LAUNCH_PC)
#undef MPG_LAUNCH_PC
    case W4A16_RING3_128x64: return launch_ring<3>(p, plan, ws, stream, lg);
    case W4A16_RING4_128x64: return launch_ring<4>(p, plan, ws, stream, lg);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w4a16(const W4A16Problem &p, const W4A16Plan &plan, const W4A16Workspace &ws,
                        hipStream_t stream) {
    int lg = 0;
    while ((1 << lg) < p.G)
        ++lg;
    return launch_one(p, plan, ws, stream, lg);
}

}  // namespace mpg
