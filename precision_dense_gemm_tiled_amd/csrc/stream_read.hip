// Plain streaming read of a device buffer: the measured ceiling for a kernel
// that must read the same bytes once from cold memory (the weight-only
// decode GEMM reads 8.67 MB per call at M = 1). Calibrating the attainable
// ceiling on the card itself, instead of quoting the nominal bandwidth, is
// the measurement method of "Warp-Specialized Kernel Implementation for W4A4
// MatMul on Latest GPU Architectures", section 2.
//
// Each thread issues all its 16-byte loads (LPL per lane, consecutive lanes
// on consecutive 16-byte chunks) before it combines any, XOR-folds them and
// the workgroup writes one word, so no load can be removed.
#include <hip/hip_runtime.h>

#include "mpgemm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int LPL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *src, int64_t chunks, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 v[LPL];
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
        const int64_t c = first + i * stride;
        v[i] = c < chunks ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0u;
#pragma unroll
    for (int i = 0; i < LPL; ++i)
        x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    // workgroup XOR through a butterfly over the wavefront and LDS
    for (int o = 32; o > 0; o >>= 1)
        x ^= __shfl_xor(x, o);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" mpgemm_status_t mpgemm_stream_read(const void *src, int64_t bytes, int loads_per_lane,
                                              uint32_t *sink, int64_t sink_words, void *stream) {
    if (bytes < 0 || !sink || (bytes > 0 && !src))
        return MPGEMM_ERR_INVALID_ARG;
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
        return MPGEMM_ERR_UNSUPPORTED;
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    const int64_t chunks = bytes / 16;
    const int64_t per_block = 256LL * loads_per_lane;
    const int64_t blocks = chunks == 0 ? 1 : (chunks + per_block - 1) / per_block;
    if (blocks > sink_words || blocks > 0x7FFFFFFF)
        return MPGEMM_ERR_INVALID_ARG;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(256);
    switch (loads_per_lane) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, st, s, chunks, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, st, s, chunks, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, st, s, chunks, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, st, s, chunks, sink); break;
    }
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}
