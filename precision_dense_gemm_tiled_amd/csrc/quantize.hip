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
// bit-identical to the exact-arithmetic definition (the codes: see below). Each lane stores its 8
// codes of a row as one 32-bit word (low nibble = even k), the first lane of
// each group stores the scale. HBM-bound: 2.5 bytes per weight plus the
// scales, so the per-weight arithmetic avoids a division.
#include "mpgemm_internal.h"

namespace mpg {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Grid: x = groups of RPW rows, y = blocks of 4 segments of 512 k (one per
// wavefront; a wave-uniform loop covers segments past 4 * gridDim.y). RPW rows
// per wavefront: their loads are all issued before any arithmetic, so each
// wavefront keeps RPW x 1 KiB in flight.
template <int RPW>
__global__ __launch_bounds__(256) void quantize_w4_kernel(QuantizeW4Problem p, int segs, int lg) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n0 = blockIdx.x * RPW;
    const int lpg = 1 << (lg - 3);   // lanes per group: G / 8, 4 ... 64
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
            float w[8];
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t bits = (uint16_t)((uint32_t)v[i][e / 2] >> (16 * (e % 2)));
                w[e] = (float)__builtin_bit_cast(_Float16, bits);
                amax = fmaxf(amax, fabsf(w[e]));
            }
            // group maximum over lpg consecutive lanes (groups are aligned; every
            // lane of the wavefront takes part, lanes past K with zeros)
            for (int o = 1; o < lpg; o <<= 1)
                amax = fmaxf(amax, __shfl_xor(amax, o));

            const _Float16 s16 = (_Float16)(amax / 7.0f);
            const float s = (float)s16;
            // q = round_half_even(w / s) without a division per weight. For
            // binary16 w and s the exact quotient is either a tie (k + 1/2
            // exactly) or at least ~2^-14 away from every half-integer, while
            // w * (1/s) in fp32 is within ~2^-19 of it (also with a reciprocal
            // one ulp off): rint of the product is exact except at ties
            // (checked over all binary16 s > 0 and w with |w / s| <= 7.5).
            // A tie shows as a remainder w - q s (exact in fp32: q has at most
            // 4 bits) of exactly s / 2; an odd guess then moves to the even
            // neighbour.
            const float inv = s > 0.f ? 1.0f / s : 0.f;
            const float half = 0.5f * s;
            uint32_t packed = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float q = rintf(w[e] * inv);
                const float rem = fmaf(-q, s, w[e]);
                if (fabsf(rem) == half && ((int)q & 1) != 0)
                    q += rem > 0.f ? 1.f : -1.f;
                int qi = (int)q;
                qi = qi > 7 ? 7 : (qi < -8 ? -8 : qi);
                packed |= (uint32_t)(qi & 0xF) << (4 * e);
            }
            if (live && n < p.N) {
                *reinterpret_cast<uint32_t *>(p.Q + (int64_t)n * p.ldq_b + k0 / 2) = packed;
                if ((lane & (lpg - 1)) == 0)
                    p.S[(int64_t)n * p.lds + (k0 >> lg)] = __builtin_bit_cast(uint16_t, s16);
            }
        }
    }
}

hipError_t launch_quantize_w4(const QuantizeW4Problem &p, hipStream_t stream) {
    constexpr int RPW = 1;   // measured: 4 rows per wavefront is no faster
    const int segs = (p.K + 511) / 512;
    const int64_t row_groups = ((int64_t)p.N + RPW - 1) / RPW;
    const int seg_blocks = (segs + 3) / 4 < 65535 ? (segs + 3) / 4 : 65535;
    if (row_groups > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    int lg = 0;
    while ((1 << lg) < p.G)
        ++lg;
    hipLaunchKernelGGL((quantize_w4_kernel<RPW>), dim3((unsigned)row_groups, seg_blocks), dim3(256), 0, stream,
                       p, segs, lg);
    return hipGetLastError();
}

}  // namespace mpg
