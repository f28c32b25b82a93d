// Symmetric round-to-nearest INT4 quantisation of fp16 weights per
// (row, G-wide K group): the step that produces the packed weights and the
// fp16 scales the weight-only GEMM consumes ("fused-int4-gemm-sm75" README,
// feature list: per-group scaling factors with group_size = 128 and packed
// INT4 weights; the page names no formula, so the plainest symmetric reading):
//   s = fp16_rne(max_k |w| / 7)
//   q = clamp(round_half_even(w / s), -8, 7), q = 0 when s == 0
//
// One wavefront covers 512 consecutive k of a row: lane l owns 8 weights
// (one 16-byte load), a group is G / 8 consecutive lanes and its maximum is
// taken with DPP lane moves inside 16-lane rows (and shuffles for G >= 256).
// Each lane stores its 8 codes as one 32-bit word (low nibble = even k), the
// first lane of each group stores the scale. 2.5 bytes per weight plus the
// scales: the kernel is meant to stream, so the arithmetic per weight is kept
// to a handful of operations, all exact:
//
// - the scale is fp16(fp32(amax) * fp32(1/7)), which equals rounding the
//   exact quotient amax / 7 once for every binary16 amax;
// - the code: for binary16 w and s the exact quotient w / s is either a tie
//   (k + 1/2 exactly) or at least ~2^-14 away from every half-integer, and
//   w * r with r the hardware reciprocal of s (within one fp32 ulp) is within
//   2^-19 of it. One fused multiply-add y = fma(w, r, 192) rounds w * r once
//   to the 2^-16 grid of [128, 256): ties land on k + 1/2 exactly and nothing
//   else crosses a half-integer. y is clamped to [184, 199] (codes -8 ... 7;
//   |w / s| can exceed 7.5 only for subnormal scales), and y + (1.5 * 2^23 +
//   8 - 192) rounds half to even to the integer 1.5 * 2^23 + q + 8, whose low
//   byte is q + 8. Two codes per byte with one shift-or, two bytes per half
//   word with another, one byte permute for the word and one XOR with
//   0x88888888 (q + 8 -> q & 15) pack the 8 codes.
// These steps are replayed against exact arithmetic, over every binary16
// scale and the weights at and next to every tie and integer multiple, in
// the CPU tests of the quantiser's arithmetic.
#include "mpgemm_internal.h"

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// maximum over LPG consecutive lanes (LPG a power of two, aligned groups)
template <int LPG>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (LPG >= 2)
        v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm 1,0,3,2
    if constexpr (LPG >= 4)
        v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm 2,3,0,1
    if constexpr (LPG >= 8)
        v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror (8 lanes)
    if constexpr (LPG >= 16)
        v = fmaxf(v, dpp_mov<0x140>(v));   // row_mirror (16 lanes)
    if constexpr (LPG >= 32)
        v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (LPG >= 64)
        v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Grid: x = groups of RPW rows, y = blocks of 4 segments of 512 k (one per
// wavefront; a wave-uniform loop covers segments past 4 * gridDim.y). The
// loads of the RPW rows are issued before any arithmetic. LPG = G / 8.
template <int LPG, int RPW>
__global__ __launch_bounds__(256) void quantize_w4_kernel(QuantizeW4Problem p, int segs, int lg) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n0 = blockIdx.x * RPW;
    for (int seg = blockIdx.y * 4 + wv; seg < segs; seg += gridDim.y * 4) {
        const int k0 = seg * 512 + 8 * lane;
        const bool live = k0 < p.K;
        i32x4 v[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int n = min(n0 + i, p.N - 1);
            v[i] = live ? *reinterpret_cast<const i32x4 *>(p.W + (int64_t)n * p.ldw + k0) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int n = n0 + i;
            // |w| as packed fp16 (sign bits cleared), then the maximum of the 8
            f16x2 h[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                h[d] = __builtin_bit_cast(f16x2, (uint32_t)v[i][d] & 0x7FFF7FFFu);
            const f16x2 m2 = __builtin_elementwise_max(__builtin_elementwise_max(h[0], h[1]),
                                                       __builtin_elementwise_max(h[2], h[3]));
            const float amax = group_max<LPG>(fmaxf((float)m2[0], (float)m2[1]));

            const _Float16 s16 = (_Float16)(amax * (1.0f / 7.0f));
            const float s = (float)s16;
            const float r = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
            uint32_t u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const _Float16 w = __builtin_bit_cast(_Float16, (uint16_t)((uint32_t)v[i][e / 2] >> (16 * (e % 2))));
                const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf((float)w, r, 192.0f), 184.0f, 199.0f);
                u[e] = __builtin_bit_cast(uint32_t, y + 12582728.0f);   // low byte: q + 8
            }
            const uint32_t b01 = (u[1] << 4) | u[0], b23 = (u[3] << 4) | u[2];
            const uint32_t b45 = (u[5] << 4) | u[4], b67 = (u[7] << 4) | u[6];
            const uint32_t lo = (b23 << 8) | b01, hi = (b67 << 8) | b45;
            const uint32_t packed = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x88888888u;
            if (live && n < p.N) {
                *reinterpret_cast<uint32_t *>(p.Q + (int64_t)n * p.ldq_b + k0 / 2) = packed;
                if ((lane & (LPG - 1)) == 0)
                    p.S[(int64_t)n * p.lds + (k0 >> lg)] = __builtin_bit_cast(uint16_t, s16);
            }
        }
    }
}

template <int RPW>
static hipError_t launch_quantize_rpw(const QuantizeW4Problem &p, hipStream_t stream, int segs, int seg_blocks,
                                      int lg) {
    const dim3 grid((unsigned)((p.N + RPW - 1) / RPW), seg_blocks);
    switch (lg) {
    case 5: hipLaunchKernelGGL((quantize_w4_kernel<4, RPW>), grid, dim3(256), 0, stream, p, segs, lg); break;
    case 6: hipLaunchKernelGGL((quantize_w4_kernel<8, RPW>), grid, dim3(256), 0, stream, p, segs, lg); break;
    case 7: hipLaunchKernelGGL((quantize_w4_kernel<16, RPW>), grid, dim3(256), 0, stream, p, segs, lg); break;
    case 8: hipLaunchKernelGGL((quantize_w4_kernel<32, RPW>), grid, dim3(256), 0, stream, p, segs, lg); break;
    case 9: hipLaunchKernelGGL((quantize_w4_kernel<64, RPW>), grid, dim3(256), 0, stream, p, segs, lg); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_w4(const QuantizeW4Problem &p, hipStream_t stream) {
    const int segs = (p.K + 511) / 512;
    const int seg_blocks = (segs + 3) / 4 < 65535 ? (segs + 3) / 4 : 65535;
    if (p.N > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int lg = 0;
    while ((1 << lg) < p.G)
        ++lg;
    // two rows per wavefront: 4096 x 4096 9.48 us against 10.08 with one and
    // 9.73 with four; 8192 x 8192 31.1, 31.4 and 33.6 us
    return launch_quantize_rpw<2>(p, stream, segs, seg_blocks, lg);
}

}  // namespace mpg
