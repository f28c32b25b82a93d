// Symmetric round-to-nearest INT4 quantisation of fp16 weights per
// (row, G-wide K group): the step that produces the packed weights and the
// fp16 scales the weight-only GEMM consumes ("fused-int4-gemm-sm75" README,
// feature list: per-group scaling factors with group_size = 128 and packed
// INT4 weights; the page names no formula, so the plainest symmetric reading):
//   s = fp16_rne(max_k |w| / 7)
//   q = clamp(round_half_even(w / s), -8, 7), q = 0 when s == 0
//
// One wavefront covers 512 consecutive k of RPW rows: lane l owns 8 weights
// of each row (one 16-byte load per row), a group is G / 8 consecutive lanes,
// the group maximum is a butterfly over those lanes. The scale is the correctly rounded fp32
// quotient rounded to fp16; for binary16 inputs that equals rounding the exact
// quotient (checked over every fp16 value), so scales and codes are
// bit-identical to the exact-arithmetic definition. Each lane stores its 8
// codes of a row as one 32-bit word (low nibble = even k), the first lane of
// each group stores the scale. HBM-bound: 2.5 bytes per weight plus the
// scales, so the per-weight arithmetic avoids a division.
#include "mpgemm_internal.h"

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// RPW rows per wavefront: their loads are all issued before any arithmetic,
// so each wavefront keeps RPW x 1 KiB in flight.
template <int RPW>
__global__ __launch_bounds__(256) void quantize_w4_kernel(QuantizeW4Problem p, int segs, int lanes_per_group) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t row_groups = ((int64_t)p.N + RPW - 1) / RPW;
    if (wid >= row_groups * segs)
        return;   // whole wavefronts only: the butterfly below stays inside live wavefronts
    const int n0 = (int)(wid / segs) * RPW, seg = (int)(wid % segs);
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
        float w[8];
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t bits = (uint16_t)((uint32_t)v[i][e / 2] >> (16 * (e % 2)));
            w[e] = (float)__builtin_bit_cast(_Float16, bits);
            amax = fmaxf(amax, fabsf(w[e]));
        }
        // group maximum over lanes_per_group consecutive lanes (groups are aligned)
        for (int o = 1; o < lanes_per_group; o <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o));

        const _Float16 s16 = (_Float16)(amax / 7.0f);
        const float s = (float)s16;
        // q = round_half_even(w / s) without a division per weight: a first
        // guess from the reciprocal (within 0.5 + 1 ulp of the quotient), then
        // the remainder w - q s, which is exact in fp32 for binary16 w and s
        // (q has at most 4 bits), decides the rounding exactly, ties to even
        // included
        const float inv = s > 0.f ? 1.0f / s : 0.f;
        const float half = 0.5f * s;
        uint32_t packed = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = rintf(w[e] * inv);
            const float rem = fmaf(-q, s, w[e]);
            const bool odd = ((int)q & 1) != 0;
            q += (rem > half || (rem == half && odd)) ? 1.f : 0.f;
            q -= (rem < -half || (rem == -half && odd)) ? 1.f : 0.f;
            int qi = s > 0.f ? (int)q : 0;
            qi = qi > 7 ? 7 : (qi < -8 ? -8 : qi);
            packed |= (uint32_t)(qi & 0xF) << (4 * e);
        }
        if (live && n < p.N) {
            *reinterpret_cast<uint32_t *>(p.Q + (int64_t)n * p.ldq_b + k0 / 2) = packed;
            if (lane % lanes_per_group == 0)
                p.S[(int64_t)n * p.lds + k0 / p.G] = __builtin_bit_cast(uint16_t, s16);
        }
    }
}

hipError_t launch_quantize_w4(const QuantizeW4Problem &p, hipStream_t stream) {
    constexpr int RPW = 1;   // measured: 4 rows per wavefront is no faster
    const int segs = (p.K + 511) / 512;
    const int64_t waves = ((int64_t)p.N + RPW - 1) / RPW * segs;
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_w4_kernel<RPW>), dim3((unsigned)blocks), dim3(256), 0, stream, p, segs, p.G / 8);
    return hipGetLastError();
}

}  // namespace mpg
