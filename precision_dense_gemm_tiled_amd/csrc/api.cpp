// C-ABI of libmpgemm: handles, argument validation and kernel dispatch.
// The public contract (argument meaning, layouts, ownership, errors) is
// documented in include/mpgemm.h; this file enforces it before any HIP call.
#include "mpgemm.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <cstring>
#include <new>

#include "mpgemm_internal.h"

struct mpgemm_ctx {
    int device;
    int cu_count;
    int forced_tile_cfg;   // -1: heuristic; else a TileCfg index (MPGEMM_TILE_CFG)
    int forced_w4a16_cfg;  // -1: heuristic; else a W4A16Cfg index (MPGEMM_W4A16_CFG)
    int streamk_mode;      // mpg::StreamKMode (MPGEMM_STREAMK=0/1 forces it off/on)
    // One device buffer of partial sums, used by the weight-only path's K
    // split and by stream-K tile GEMMs (calls sharing a handle are serialized
    // by the caller), and the stream-K arrival counters (zero between calls).
    mpg::W4A16Workspace ws;
    mpg::TileWorkspace tile_ws;
};

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of a C = A * B^T call. elem_num/elem_den: bytes per element
// of A and B (1/2 for packed INT4); out_bytes: bytes per element of C.
// Every argument check of a GEMM call except the handle.
mpgemm_status_t check_gemm_args(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                const void *B, int64_t ldb, const void *C, int64_t ldc, int elem_num,
                                int elem_den, int out_bytes, int64_t max_k, bool *noop) {
    *noop = false;
    if (M < 0 || N < 0 || K < 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        *noop = true;
        return MPGEMM_OK;
    }
    if (!C || (K > 0 && (!A || !B)))
        return MPGEMM_ERR_INVALID_ARG;
    if (lda < K || ldb < K || ldc < N)
        return MPGEMM_ERR_INVALID_ARG;
    if (M > INT_MAX || N > INT_MAX || K > max_k)
        return MPGEMM_ERR_UNSUPPORTED;
    // the tile kernel flattens the tile grid into one 32-bit dimension
    if (((M + 63) / 64) * ((N + 63) / 64) > INT_MAX)
        return MPGEMM_ERR_UNSUPPORTED;
    if ((lda * elem_num) % elem_den != 0 || (ldb * elem_num) % elem_den != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    // C is written one element at a time: element alignment suffices. A and B
    // may have any alignment (rows that are not 16-byte aligned take a slower
    // byte-gather kernel).
    if ((reinterpret_cast<uintptr_t>(C) % out_bytes) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    return MPGEMM_OK;
}

// The handle is checked last so that every argument error is reported without
// a device (and can be tested on a host without a GPU).
mpgemm_status_t check_gemm(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K, const void *A,
                           int64_t lda, const void *B, int64_t ldb, const void *C, int64_t ldc,
                           int elem_num, int elem_den, int out_bytes, int64_t max_k, bool *noop) {
    mpgemm_status_t st =
        check_gemm_args(M, N, K, A, lda, B, ldb, C, ldc, elem_num, elem_den, out_bytes, max_k, noop);
    if (st != MPGEMM_OK || *noop)
        return st;
    return h ? MPGEMM_OK : MPGEMM_ERR_INVALID_ARG;
}

// Partial-sum workspace per handle: 128 MiB (two 256 x 256 fp32 tiles per
// compute unit for stream-K); the weight-only K split uses its first 32 MiB.
constexpr int64_t kWorkspaceBytes = int64_t(128) << 20;
constexpr int64_t kSplitPartialFloats = int64_t(8) << 20;
// Stream-K arrival counters: one per split tile (at most two waves of tiles).
constexpr int kStreamKFlags = 16384;

// Makes the handle's device current for the duration of a call and restores
// the caller's current device afterwards.
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int device) {
        if (hipGetDevice(&prev) != hipSuccess) {
            prev = -1;
            return;
        }
        ok = prev == device || hipSetDevice(device) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev)
            (void)hipSetDevice(prev);
    }
};

// The low-rank branch of a W4A4 call: U (fp32, M x rank) and the up-projection.
struct LowRankArgs {
    const float *u;
    const uint16_t *v;
    int64_t ldu, ldv;
    int rank;
};

mpgemm_status_t run_tile(mpgemm_handle_t h, int prec, int64_t M, int64_t N, int64_t kbytes,
                         const void *A, int64_t lda_b, const void *B, int64_t ldb_b, void *C,
                         int64_t ldc, void *stream, const uint16_t *sx = nullptr,
                         const uint16_t *sw = nullptr, const uint16_t *bias = nullptr,
                         const LowRankArgs *lr = nullptr, const mpg::TileWorkspace *ws = nullptr) {
    DeviceGuard dg(h->device);
    if (!dg.ok)
        return MPGEMM_ERR_HIP;
    mpg::GemmProblem p;
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.C = C;
    p.lda_b = lda_b;
    p.ldb_b = ldb_b;
    p.ldc = ldc;
    p.M = (int)M;
    p.N = (int)N;
    p.kbytes = kbytes;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.c_vec16 = (reinterpret_cast<uintptr_t>(C) % 16 == 0 && ldc % 4 == 0) ? 1 : 0;
    if (lr) {
        p.lr_u = lr->u;
        p.lr_v = lr->v;
        p.lr_ldu = lr->ldu;
        p.lr_ldv = lr->ldv;
        p.lr_rank = lr->rank;
    }
    const mpg::TileWorkspace &tws = ws ? *ws : h->tile_ws;
    int cfg = h->forced_tile_cfg >= 0 ? h->forced_tile_cfg
                                      : mpg::choose_tile_cfg(prec, M, N, kbytes, h->cu_count);
    const mpg::StreamKPlan sk =
        mpg::plan_stream_k(cfg, M, N, kbytes, h->cu_count, tws.partial_bytes, tws.flag_count,
                           h->streamk_mode);
    hipError_t e = mpg::launch_gemm(prec, cfg, p, sk, tws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

// Checks of a transposed-B call: B^T is K x N (row stride ldbt elements).
// That kernel has no byte-gather variant, so A and B^T rows must be 16-byte
// aligned. The handle is checked last, as for the other calls.
mpgemm_status_t check_gemm_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K, const void *A,
                              int64_t lda, const void *Bt, int64_t ldbt, const void *C, int64_t ldc,
                              int elem_num, int elem_den, int out_bytes, int64_t max_k, bool *noop) {
    *noop = false;
    if (M < 0 || N < 0 || K < 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        *noop = true;
        return MPGEMM_OK;
    }
    if (!C || (K > 0 && (!A || !Bt)))
        return MPGEMM_ERR_INVALID_ARG;
    if (lda < K || ldbt < N || ldc < N)
        return MPGEMM_ERR_INVALID_ARG;
    if (M > INT_MAX || N > INT_MAX || K > max_k || lda > INT64_MAX / 4 || ldbt > INT64_MAX / 4)
        return MPGEMM_ERR_UNSUPPORTED;
    if (((M + 255) / 256) * ((N + 255) / 256) > INT_MAX)
        return MPGEMM_ERR_UNSUPPORTED;
    if ((lda * elem_num) % elem_den != 0 || (ldbt * elem_num) % elem_den != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    // (K == 0 reads no operand: it writes zeros whatever the layout)
    if (K > 0 && ((lda * elem_num / elem_den) % 16 != 0 || (ldbt * elem_num / elem_den) % 16 != 0 ||
                  !aligned16(A) || !aligned16(Bt)))
        return MPGEMM_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(C) % out_bytes) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    return h ? MPGEMM_OK : MPGEMM_ERR_INVALID_ARG;
}

mpgemm_status_t run_kn(mpgemm_handle_t h, int prec, int64_t M, int64_t N, int64_t kbytes,
                       const void *A, int64_t lda_b, const void *Bt, int64_t ldbt_b, void *C,
                       int64_t ldc, void *stream) {
    DeviceGuard dg(h->device);
    if (!dg.ok)
        return MPGEMM_ERR_HIP;
    mpg::GemmProblem p;
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(Bt);
    p.C = C;
    p.lda_b = lda_b;
    p.ldb_b = ldbt_b;
    p.ldc = ldc;
    p.M = (int)M;
    p.N = (int)N;
    p.kbytes = kbytes;
    p.sx = p.sw = p.bias = nullptr;
    p.c_vec16 = 0;
    hipError_t e = mpg::launch_gemm_kn(prec, p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

}  // namespace

namespace mpg {

// Every argument check of a weight-only call except the handle (shared with
// the allocation-free entry point).
mpgemm_status_t check_w4a16_args(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                                 const uint8_t *Wq, int64_t ldw, const uint16_t *S, int64_t lds,
                                 int64_t group_size, const uint16_t *Y, int64_t ldy, bool *noop) {
    *noop = false;
    if (M < 0 || N < 0 || K < 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        *noop = true;
        return MPGEMM_OK;
    }
    if (!Y || (K > 0 && (!X || !Wq || !S)))
        return MPGEMM_ERR_INVALID_ARG;
    if (ldx < K || ldw < K || ldy < N)
        return MPGEMM_ERR_INVALID_ARG;
    const bool pow2 = group_size > 0 && (group_size & (group_size - 1)) == 0;
    if (K > 0) {
        if (!pow2 || group_size < 32 || group_size > K || K % group_size != 0)
            return MPGEMM_ERR_UNSUPPORTED;
        if (lds < K / group_size)
            return MPGEMM_ERR_INVALID_ARG;
    }
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX || (M + 31) / 32 > 65535)
        return MPGEMM_ERR_UNSUPPORTED;
    if ((ldw % 2) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    if ((K > 0 && (!aligned16(X) || !aligned16(Wq) || (reinterpret_cast<uintptr_t>(S) & 1u))) ||
        (reinterpret_cast<uintptr_t>(Y) & 1u))
        return MPGEMM_ERR_UNSUPPORTED;
    if ((ldx * 2) % 16 != 0 || (ldw / 2) % 16 != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    return MPGEMM_OK;
}

W4A16Problem make_w4a16_problem(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                                const uint8_t *Wq, int64_t ldw, const uint16_t *S, int64_t lds,
                                int64_t group_size, uint16_t *Y, int64_t ldy) {
    W4A16Problem p;
    p.X = X;
    p.W = Wq;
    p.S = S;
    p.Y = Y;
    p.ldx = ldx;
    p.ldw_b = ldw / 2;
    p.lds = lds;
    p.ldy = ldy;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.G = K > 0 ? (int)group_size : 32;
    return p;
}

int64_t w4a16_split_floats() { return kSplitPartialFloats; }

}  // namespace mpg

extern "C" {

mpgemm_status_t mpgemm_create(mpgemm_handle_t *out, int device) {
    if (!out)
        return MPGEMM_ERR_INVALID_ARG;
    *out = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
        return MPGEMM_ERR_DEVICE;
    if (device < 0) {
        if (hipGetDevice(&device) != hipSuccess)
            return MPGEMM_ERR_DEVICE;
    }
    if (device >= count)
        return MPGEMM_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess)
        return MPGEMM_ERR_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return MPGEMM_ERR_DEVICE;
    mpgemm_ctx *h = new (std::nothrow) mpgemm_ctx;
    if (!h)
        return MPGEMM_ERR_HIP;
    h->device = device;
    h->cu_count = prop.multiProcessorCount;
    h->forced_tile_cfg = -1;
    // One-parameter-at-a-time ablations: force a tile configuration by index.
    if (const char *env = std::getenv("MPGEMM_TILE_CFG")) {
        int v = std::atoi(env);
        if (v >= 0 && v < mpg::CFG_COUNT)
            h->forced_tile_cfg = v;
    }
    h->forced_w4a16_cfg = -1;
    if (const char *env = std::getenv("MPGEMM_W4A16_CFG")) {
        int v = std::atoi(env);
        if (v >= 0 && v < mpg::W4A16_CFG_COUNT)
            h->forced_w4a16_cfg = v;
    }
    h->streamk_mode = mpg::SK_MODE_AUTO;
    if (const char *env = std::getenv("MPGEMM_STREAMK")) {
        if (env[0] == '0')
            h->streamk_mode = mpg::SK_MODE_OFF;
        else if (env[0] == '1')
            h->streamk_mode = mpg::SK_MODE_ON;
        else if (env[0] == '2')
            h->streamk_mode = mpg::SK_MODE_PERSIST;
    }
    // Workspace (partial sums of split K loops, stream-K arrival counters),
    // allocated once here; the counters start at zero and every stream-K
    // launch leaves them at zero.
    h->ws.partial = nullptr;
    h->ws.partial_floats = kSplitPartialFloats;
    h->tile_ws.partial = nullptr;
    h->tile_ws.partial_bytes = kWorkspaceBytes;
    h->tile_ws.flags = nullptr;
    h->tile_ws.flag_count = kStreamKFlags;
    int prev = -1;
    bool ok = hipGetDevice(&prev) == hipSuccess && hipSetDevice(device) == hipSuccess;
    ok = ok && hipMalloc(&h->tile_ws.partial, kWorkspaceBytes) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&h->tile_ws.flags), kStreamKFlags * sizeof(int)) == hipSuccess;
    ok = ok && hipMemset(h->tile_ws.flags, 0, kStreamKFlags * sizeof(int)) == hipSuccess;
    ok = ok && hipDeviceSynchronize() == hipSuccess;
    h->ws.partial = static_cast<float *>(h->tile_ws.partial);
    if (prev >= 0)
        (void)hipSetDevice(prev);
    if (!ok) {
        mpgemm_destroy(h);
        return MPGEMM_ERR_HIP;
    }
    *out = h;
    return MPGEMM_OK;
}

mpgemm_status_t mpgemm_destroy(mpgemm_handle_t h) {
    if (!h)
        return MPGEMM_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    if (h->tile_ws.partial)
        (void)hipFree(h->tile_ws.partial);
    if (h->tile_ws.flags)
        (void)hipFree(h->tile_ws.flags);
    if (prev >= 0)
        (void)hipSetDevice(prev);
    delete h;
    return MPGEMM_OK;
}

const char *mpgemm_status_string(mpgemm_status_t s) {
    switch (s) {
    case MPGEMM_OK: return "MPGEMM_OK";
    case MPGEMM_ERR_INVALID_ARG: return "MPGEMM_ERR_INVALID_ARG";
    case MPGEMM_ERR_UNSUPPORTED: return "MPGEMM_ERR_UNSUPPORTED";
    case MPGEMM_ERR_DEVICE: return "MPGEMM_ERR_DEVICE";
    case MPGEMM_ERR_HIP: return "MPGEMM_ERR_HIP";
    default: return "MPGEMM_UNKNOWN_STATUS";
    }
}

mpgemm_status_t mpgemm_run_f16(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                               float *C, int64_t ldc, void *stream) {
    bool noop;
    mpgemm_status_t st = check_gemm(h, M, N, K, A, lda, B, ldb, C, ldc, 2, 1, 4, INT64_MAX / 4, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_tile(h, mpg::PREC_F16, M, N, 2 * K, A, 2 * lda, B, 2 * ldb, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_i8(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                              const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                              int32_t *C, int64_t ldc, void *stream) {
    bool noop;
    mpgemm_status_t st =
        check_gemm(h, M, N, K, A, lda, B, ldb, C, ldc, 1, 1, 4, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_tile(h, mpg::PREC_I8, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_i4(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                              const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                              int32_t *C, int64_t ldc, void *stream) {
    if (M > 0 && N > 0 && K >= 0 && ((K % 2) != 0 || (lda % 2) != 0 || (ldb % 2) != 0))
        return MPGEMM_ERR_UNSUPPORTED;
    bool noop;
    mpgemm_status_t st =
        check_gemm(h, M, N, K, A, lda, B, ldb, C, ldc, 1, 2, 4, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_tile(h, mpg::PREC_I4, M, N, K / 2, A, lda / 2, B, ldb / 2, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_f16_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                  const uint16_t *A, int64_t lda, const uint16_t *Bt, int64_t ldbt,
                                  float *C, int64_t ldc, void *stream) {
    bool noop;
    mpgemm_status_t st =
        check_gemm_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, 2, 1, 4, INT64_MAX / 4, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_kn(h, mpg::PREC_F16, M, N, 2 * K, A, 2 * lda, Bt, 2 * ldbt, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_i8_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const int8_t *A, int64_t lda, const int8_t *Bt, int64_t ldbt,
                                 int32_t *C, int64_t ldc, void *stream) {
    bool noop;
    mpgemm_status_t st =
        check_gemm_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, 1, 1, 4, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_kn(h, mpg::PREC_I8, M, N, K, A, lda, Bt, ldbt, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_i4_kn(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const uint8_t *A, int64_t lda, const uint8_t *Bt, int64_t ldbt,
                                 int32_t *C, int64_t ldc, void *stream) {
    if (M > 0 && N > 0 && K >= 0 && ((K % 2) != 0 || (lda % 2) != 0 || (ldbt % 2) != 0))
        return MPGEMM_ERR_UNSUPPORTED;
    bool noop;
    mpgemm_status_t st =
        check_gemm_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, 1, 2, 4, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    return run_kn(h, mpg::PREC_I4, M, N, K / 2, A, lda / 2, Bt, ldbt / 2, C, ldc, stream);
}

mpgemm_status_t mpgemm_run_w4a4(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                const uint16_t *SX, const uint16_t *SW, const uint16_t *bias,
                                uint16_t *Y, int64_t ldy, void *stream) {
    if (M > 0 && N > 0 && K >= 0 && ((K % 2) != 0 || (lda % 2) != 0 || (ldb % 2) != 0))
        return MPGEMM_ERR_UNSUPPORTED;
    bool noop;
    mpgemm_status_t st =
        check_gemm_args(M, N, K, A, lda, B, ldb, Y, ldy, 1, 2, 2, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    if (!SX || !SW)
        return MPGEMM_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(SX) | reinterpret_cast<uintptr_t>(SW) |
         reinterpret_cast<uintptr_t>(bias)) & 1u)
        return MPGEMM_ERR_UNSUPPORTED;
    if (!h)
        return MPGEMM_ERR_INVALID_ARG;
    return run_tile(h, mpg::PREC_W4A4, M, N, K / 2, A, lda / 2, B, ldb / 2, Y, ldy, stream, SX, SW, bias);
}

mpgemm_status_t mpgemm_run_w4a4_lowrank(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                        const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                        const uint16_t *SX, const uint16_t *SW, const uint16_t *bias,
                                        const uint16_t *X, int64_t ldx, const uint16_t *LD, int64_t ldd,
                                        const uint16_t *LU, int64_t ldu, int64_t R,
                                        uint16_t *Y, int64_t ldy, void *stream) {
    if (R == 0)
        return mpgemm_run_w4a4(h, M, N, K, A, lda, B, ldb, SX, SW, bias, Y, ldy, stream);
    if (M > 0 && N > 0 && K >= 0 && ((K % 2) != 0 || (lda % 2) != 0 || (ldb % 2) != 0))
        return MPGEMM_ERR_UNSUPPORTED;
    bool noop;
    mpgemm_status_t st =
        check_gemm_args(M, N, K, A, lda, B, ldb, Y, ldy, 1, 2, 2, MPGEMM_MAX_K_INT, &noop);
    if (st != MPGEMM_OK || noop)
        return R < 0 ? MPGEMM_ERR_INVALID_ARG : st;
    if (!SX || !SW || R < 0 || !LU || (K > 0 && (!X || !LD)) || ldx < K || ldd < K || ldu < R)
        return MPGEMM_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(SX) | reinterpret_cast<uintptr_t>(SW) |
         reinterpret_cast<uintptr_t>(bias) | reinterpret_cast<uintptr_t>(X) |
         reinterpret_cast<uintptr_t>(LD)) & 1u)
        return MPGEMM_ERR_UNSUPPORTED;
    // the epilogue reads LU rows with 16-byte loads, 16 of rank per step
    if (R % 16 != 0 || R > MPGEMM_MAX_LOWRANK || !aligned16(LU) || ldu % 8 != 0 ||
        ldx > INT64_MAX / 4 || ldd > INT64_MAX / 4 || ldu > INT64_MAX / 4)
        return MPGEMM_ERR_UNSUPPORTED;
    if (!h)
        return MPGEMM_ERR_INVALID_ARG;
    // U = X LD^T (fp32, M x R) at the start of the handle's workspace; the
    // stream-K partials of both launches get the rest
    const int64_t ubytes = (M * R * 4 + 255) / 256 * 256;
    if (ubytes > h->tile_ws.partial_bytes / 2)
        return MPGEMM_ERR_UNSUPPORTED;
    float *U = static_cast<float *>(h->tile_ws.partial);
    mpg::TileWorkspace rest = h->tile_ws;
    rest.partial = static_cast<uint8_t *>(h->tile_ws.partial) + ubytes;
    rest.partial_bytes = h->tile_ws.partial_bytes - ubytes;
    if (K > 0 && K % 64 == 0 && R <= 64 && aligned16(X) && aligned16(LD) && ldx % 8 == 0 && ldd % 8 == 0 &&
        h->forced_tile_cfg < 0) {
        // the skinny down-projection kernel (X read once, coalesced)
        DeviceGuard dg(h->device);
        if (!dg.ok)
            return MPGEMM_ERR_HIP;
        const mpg::LowRankDown d{X, LD, U, ldx, ldd, R, (int)M, (int)K, (int)R};
        if (mpg::launch_lowrank_down(d, static_cast<hipStream_t>(stream)) != hipSuccess)
            return MPGEMM_ERR_HIP;
    } else {
        // other layouts and ranks, or a forced tile configuration: the FP16 tile GEMM
        st = run_tile(h, mpg::PREC_F16, M, R, 2 * K, X, 2 * ldx, LD, 2 * ldd, U, R, stream, nullptr, nullptr,
                      nullptr, nullptr, &rest);
        if (st != MPGEMM_OK)
            return st;
    }
    const LowRankArgs lr{U, LU, R, ldu, (int)R};
    return run_tile(h, mpg::PREC_W4A4, M, N, K / 2, A, lda / 2, B, ldb / 2, Y, ldy, stream, SX, SW, bias,
                    &lr, &rest);
}

mpgemm_status_t mpgemm_run_w4a16(mpgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                 const uint16_t *X, int64_t ldx, const uint8_t *Wq, int64_t ldw,
                                 const uint16_t *S, int64_t lds, int64_t group_size,
                                 uint16_t *Y, int64_t ldy, void *stream) {
    bool noop;
    mpgemm_status_t st = mpg::check_w4a16_args(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, &noop);
    if (st != MPGEMM_OK || noop)
        return st;
    if (!h)
        return MPGEMM_ERR_INVALID_ARG;
    DeviceGuard dg(h->device);
    if (!dg.ok)
        return MPGEMM_ERR_HIP;
    const mpg::W4A16Problem p = mpg::make_w4a16_problem(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy);
    const int cfg = h->forced_w4a16_cfg >= 0 ? h->forced_w4a16_cfg : mpg::choose_w4a16_cfg(M, N, K);
    const mpg::W4A16Plan plan = mpg::plan_w4a16(M, N, K, cfg, h->cu_count, h->ws.partial_floats);
    hipError_t e = mpg::launch_w4a16(p, plan, h->ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

}  // extern "C"

mpgemm_status_t mpgemm_quantize_w4(mpgemm_handle_t h, int64_t N, int64_t K, const uint16_t *W, int64_t ldw,
                                   int64_t group_size, uint8_t *Wq, int64_t ldwq, uint16_t *S, int64_t lds,
                                   void *stream) {
    if (N < 0 || K < 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (N == 0 || K == 0)
        return MPGEMM_OK;
    if (!W || !Wq || !S)
        return MPGEMM_ERR_INVALID_ARG;
    const bool pow2 = group_size > 0 && (group_size & (group_size - 1)) == 0;
    if (!pow2 || group_size < 32 || group_size > 512 || K % group_size != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    if (ldw < K || ldwq < K || lds < K / group_size)
        return MPGEMM_ERR_INVALID_ARG;
    if (N > INT_MAX || K > INT_MAX || (ldwq % 2) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    if (!aligned16(W) || (ldw * 2) % 16 != 0 || (reinterpret_cast<uintptr_t>(Wq) & 3u) != 0 ||
        (ldwq / 2) % 4 != 0 || (reinterpret_cast<uintptr_t>(S) & 1u) != 0)
        return MPGEMM_ERR_UNSUPPORTED;
    if (!h)
        return MPGEMM_ERR_INVALID_ARG;
    DeviceGuard dg(h->device);
    if (!dg.ok)
        return MPGEMM_ERR_HIP;
    mpg::QuantizeW4Problem p;
    p.W = W;
    p.Q = Wq;
    p.S = S;
    p.ldw = ldw;
    p.ldq_b = ldwq / 2;
    p.lds = lds;
    p.N = (int)N;
    p.K = (int)K;
    p.G = (int)group_size;
    hipError_t e = mpg::launch_quantize_w4(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

mpgemm_status_t mpgemm_plan_gemm(int precision, int64_t M, int64_t N, int64_t K, int cu_count,
                                 int *config, int *sk_grid, int *sk_tiles_dp) {
    if (!config || !sk_grid || !sk_tiles_dp || M < 0 || N < 0 || K < 0 || cu_count < 1 ||
        precision < MPGEMM_PREC_F16 || precision > MPGEMM_PREC_W4A4)
        return MPGEMM_ERR_INVALID_ARG;
    const int64_t kbytes = precision == MPGEMM_PREC_F16 ? 2 * K : (precision == MPGEMM_PREC_I8 ? K : K / 2);
    *config = mpg::choose_tile_cfg(precision, M, N, kbytes, cu_count);
    const mpg::StreamKPlan sk = mpg::plan_stream_k(*config, M, N, kbytes, cu_count, kWorkspaceBytes,
                                                   kStreamKFlags, mpg::SK_MODE_AUTO);
    *sk_grid = sk.grid;
    *sk_tiles_dp = sk.tiles_dp;
    return MPGEMM_OK;
}

mpgemm_status_t mpgemm_plan_w4a16(int64_t M, int64_t N, int64_t K, int cu_count, int *config,
                                  int *k_splits, int64_t *k_slice) {
    if (!config || !k_splits || !k_slice || M < 1 || N < 1 || K < 0 || cu_count < 1)
        return MPGEMM_ERR_INVALID_ARG;
    const mpg::W4A16Plan plan =
        mpg::plan_w4a16(M, N, K, mpg::choose_w4a16_cfg(M, N, K), cu_count, kSplitPartialFloats);
    *config = plan.cfg;
    *k_splits = plan.ks;
    *k_slice = plan.ks > 1 ? plan.kslice : K;
    return MPGEMM_OK;
}
