// Weight-only INT4 GEMM for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid it):
// mpgemm_run_w4a16_noalloc. It runs the same plan and kernels as
// mpgemm_run_w4a16 with a default handle, but needs no handle: the fp32 K
// slices of a split call live in a static device array of this file, one
// copy per GPU, which every call on that GPU shares.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mpgemm.h"
#include "mpgemm_internal.h"

namespace {

// 16 MiB of fp32 partial sums per GPU, held until the process ends.
constexpr int64_t kScratchFloats = MPGEMM_NOALLOC_SCRATCH_BYTES / 4;
static __device__ __align__(256) float scratch[kScratchFloats];

// Per-device state, set up on the first call on each device with that device
// current: the device address of that GPU's copy of `scratch` (host code
// never passes the array's own name to a kernel: on the host it is a
// stand-in, not a device address) and the compute-unit count for planning.
constexpr int kMaxDevices = 64;
struct DeviceScratch {
    std::once_flag once;
    hipError_t err = hipSuccess;
    float *ptr = nullptr;
    int cu_count = 0;
};
DeviceScratch g_dev[kMaxDevices];

void init_device(DeviceScratch &d, int device) {
    void *ptr = nullptr;
    d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (d.err != hipSuccess)
        return;
    int cu = 0;
    d.err = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device);
    if (d.err != hipSuccess)
        return;
    d.ptr = static_cast<float *>(ptr);
    d.cu_count = cu;
}

}  // namespace

extern "C" mpgemm_status_t mpgemm_run_w4a16_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t *X,
                                                    int64_t ldx, const uint8_t *Wq, int64_t ldw,
                                                    const uint16_t *S, int64_t lds, int64_t group_size,
                                                    uint16_t *Y, int64_t ldy, void *stream) {
    bool noop;
    mpgemm_status_t st = mpg::check_w4a16_args(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0)
        return MPGEMM_ERR_DEVICE;
    if (device >= kMaxDevices)
        return MPGEMM_ERR_UNSUPPORTED;
    DeviceScratch &d = g_dev[device];
    std::call_once(d.once, init_device, std::ref(d), device);
    if (d.err != hipSuccess || !d.ptr)
        return MPGEMM_ERR_HIP;
    // the plan of mpgemm_run_w4a16 (handle workspace capacity), so that both
    // entry points launch the same kernels; a split that needs more than the
    // static scratch is refused
    const mpg::W4A16Plan plan =
        mpg::plan_w4a16(M, N, K, mpg::choose_w4a16_cfg(M, N, K), d.cu_count, mpg::w4a16_split_floats());
    if (mpg::w4a16_plan_scratch_floats(plan) > kScratchFloats)
        return MPGEMM_ERR_UNSUPPORTED;
    const mpg::W4A16Problem p = mpg::make_w4a16_problem(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy);
    mpg::W4A16Workspace ws;
    ws.partial = d.ptr;
    ws.partial_floats = kScratchFloats;
    const hipError_t e = mpg::launch_w4a16(p, plan, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}
