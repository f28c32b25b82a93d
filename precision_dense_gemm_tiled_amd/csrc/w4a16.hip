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

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

template <int MT, int WN, int WK, int U>
static hipError_t launch_cfg(const W4A16Problem &p, hipStream_t stream) {
    dim3 block(64 * WN * WK);
    dim3 grid((p.N + 16 * WN - 1) / (16 * WN), (p.M + 16 * MT - 1) / (16 * MT));
    int lg = 0;
    while ((1 << lg) < p.G)
        ++lg;
    // G % 128 == 0 implies K % 128 == 0: every step lies in one group
    if (p.G % 128 == 0)
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, true, true>), grid, block, 0, stream, p, lg);
    else if (p.K % 128 == 0)
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, false, true>), grid, block, 0, stream, p, lg);
    else
        hipLaunchKernelGGL((w4a16_kernel<MT, WN, WK, U, false, false>), grid, block, 0, stream, p, lg);
    return hipGetLastError();
}

hipError_t launch_w4a16(const W4A16Problem &p, hipStream_t stream) {
    if (p.M <= 16)
        return launch_cfg<1, 1, 4, 8>(p, stream);   // decode: 16 rows per workgroup, K split 4 ways
    return launch_cfg<2, 4, 1, 2>(p, stream);       // prefill: 32 x 64 tiles
}

}  // namespace mpg
