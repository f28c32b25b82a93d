// Down-projection of the W4A4 low-rank branch, U = X LD^T ("Warp-Specialized
// Kernel Implementation for W4A4 MatMul on Latest GPU Architectures",
// section 1: a small low-rank residual projection beside the 4-bit product).
// With R <= 64 ranks this is a skinny GEMM bound by reading X (M x K fp16)
// once; a square-tile GEMM leaves half of every 64-wide tile empty and half
// the chip idle at M = 8192.
//
// A workgroup owns 32 rows of X and all R ranks; its NW wavefronts take
// contiguous shares of K, 64 k per chunk. Each wavefront stages its own
// chunks (32 rows of X, 32 RB ranks of LD, 128 bytes each) in its own LDS
// slots with direct-to-LDS loads that each fetch 8 whole 128-byte row
// segments, the next chunk in flight while the current one is multiplied,
// so no barrier is needed: a wavefront only waits for its own loads. Row r's
// 16-byte chunk c sits at slot c ^ ((r / 2) & 7), so the fragment reads of
// v_mfma_f32_32x32x16_f16 (lane l: row l % 32, chunk 2 t + l / 32 of step t)
// are free of bank conflicts. The wavefronts' partial sums are added through
// LDS in wavefront order (the result does not depend on the schedule).
#include "mpgemm_internal.h"
#include "lds_dma.h"

namespace mpg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int RB, int NW>
__global__ __launch_bounds__(64 * NW) void lowrank_down_kernel(LowRankDown p) {
    constexpr int XB = 32 * 128;            // one chunk of X: 32 rows x 64 k
    constexpr int BUF = XB * (1 + RB);      // and of LD: 32 RB ranks x 64 k
    constexpr int NL = 4 * (1 + RB);        // direct-to-LDS loads per chunk
    static_assert(NL < 64, "vmcnt of the chunk wait");
    __shared__ __attribute__((aligned(16))) uint8_t lds[NW * 2 * BUF];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = blockIdx.x * 32;
    const int chunks = p.K / 64;
    const int per = (chunks + NW - 1) / NW;
    const int c0 = wave * per, c1 = min(chunks, c0 + per);
    uint8_t *mine = lds + wave * 2 * BUF;

    // load i of a 32-row block: local row 8 i + l / 8, slot l % 8 holding
    // global 16-byte chunk (l % 8) ^ ((row / 2) & 7) of the row's 128 bytes
    const int lr = lane >> 3, lq = lane & 7;
    const uint16_t *xsrc[4], *dsrc[RB][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + lr;
        const int c = lq ^ ((r >> 1) & 7);
        xsrc[i] = p.X + (int64_t)min(m0 + r, p.M - 1) * p.ldx + 8 * c;
#pragma unroll
        for (int b = 0; b < RB; ++b)   // ranks past R repeat the last (their sums are never stored)
            dsrc[b][i] = p.LD + (int64_t)min(32 * b + r, p.R - 1) * p.ldd + 8 * c;
    }
    auto issue = [&](int ch, int buf) {
        uint8_t *dst = mine + buf * BUF;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(xsrc[i] + 64 * ch, dst + 1024 * i);
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dma16(dsrc[b][i] + 64 * ch, dst + XB * (1 + b) + 1024 * i);
        asm volatile("" ::: "memory");
    };

    // fragment of step t: row l % 32, 16-byte chunk 2 t + l / 32
    const int fr = lane & 31;
    int foff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        foff[t] = fr * 128 + (((2 * t + (lane >> 5)) ^ ((fr >> 1) & 7)) * 16);

    f32x16 acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b)
        acc[b] = f32x16{};
    if (c0 < c1)
        issue(c0, 0);
    for (int c = c0; c < c1; ++c) {
        const int buf = (c - c0) & 1;
        // the slots of chunk c + 1 were last read (and consumed) in step c - 1
        if (c + 1 < c1) {
            issue(c + 1, buf ^ 1);
            wait_vm_lds<NL>();
        } else {
            wait_vm_lds<0>();
        }
        asm volatile("" ::: "memory");
        const uint8_t *src = mine + buf * BUF;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f16x8 a = *reinterpret_cast<const f16x8 *>(src + foff[t]);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const f16x8 d = *reinterpret_cast<const f16x8 *>(src + XB * (1 + b) + foff[t]);
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, d, acc[b], 0, 0, 0);
            }
        }
        asm volatile("" ::: "memory");
    }

    // register r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, rank l % 32 of the block
    static_assert(NW * 16 * 64 * 4 <= NW * 2 * BUF, "reduction buffer");
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r)
            red[(wave * 16 + r) * 64 + lane] = acc[b][r];
        __syncthreads();
        for (int e = threadIdx.x; e < 16 * 64; e += 64 * NW) {
            const int r = e / 64, l = e % 64;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                v += red[(w * 16 + r) * 64 + l];
            const int m = m0 + 8 * (r / 4) + 4 * (l / 32) + r % 4, rank = 32 * b + l % 32;
            if (m < p.M && rank < p.R)
                p.U[(int64_t)m * p.ldu + rank] = v;
        }
    }
}

template <int RB, int NW>
hipError_t launch_rb(const LowRankDown &p, hipStream_t stream) {
    const int blocks = (p.M + 31) / 32;
    hipLaunchKernelGGL((lowrank_down_kernel<RB, NW>), dim3(blocks), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_down(const LowRankDown &p, hipStream_t stream) {
    if (p.M <= 0 || p.R <= 0 || p.R > 64 || p.K <= 0 || p.K % 64 != 0)
        return hipErrorInvalidValue;
    // LDS: NW x 2 chunks of 4 KiB (1 + RB): 128 KiB at R <= 32, 96 KiB at R <= 64
    return p.R <= 32 ? launch_rb<1, 8>(p, stream) : launch_rb<2, 4>(p, stream);
}

}  // namespace mpg
