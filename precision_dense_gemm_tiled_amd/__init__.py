"""Python binding of libmpgemm (include/mpgemm.h): argument marshalling only.

The ``mpgemm_*`` functions mirror the C-ABI one to one (raw integer device
pointers and a raw ``hipStream_t``). The torch-facing helpers below them only
allocate outputs with torch, read pointers, strides and the current stream,
and call the C-ABI; every arithmetic step runs in the HIP kernels of
libmpgemm.so. There is no fallback: if the library is missing, or the device
is not a gfx950, the calls raise.
"""
import ctypes
import os

__all__ = [
    "MpgemmError", "lib", "lib_path",
    "mpgemm_create", "mpgemm_destroy", "mpgemm_status_string",
    "mpgemm_run_f16", "mpgemm_run_i8", "mpgemm_run_i4", "mpgemm_run_w4a16", "mpgemm_run_w4a4", "mpgemm_quantize_w4",
    "mpgemm_run_w4a4_lowrank", "mpgemm_run_w4a16_noalloc", "mpgemm_stream_read",
    "mpgemm_run_f16_kn", "mpgemm_run_i8_kn", "mpgemm_run_i4_kn",
    "mpgemm_plan_gemm", "mpgemm_plan_w4a16",
    "Handle", "default_handle", "gemm_f16", "gemm_i8", "gemm_i4", "gemm_w4a16", "gemm_w4a4", "gemm_w4a4_lowrank", "quantize_w4",
    "gemm_w4a16_noalloc",
    "gemm_f16_kn", "gemm_i8_kn", "gemm_i4_kn",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmpgemm.so")

MPGEMM_OK = 0
MPGEMM_ERR_INVALID_ARG = 1
MPGEMM_ERR_UNSUPPORTED = 2
MPGEMM_ERR_DEVICE = 3
MPGEMM_ERR_HIP = 4
MPGEMM_MAX_K_INT = 131071

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class MpgemmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = int(status)
        super().__init__(f"{what}: {mpgemm_status_string(status)} ({status})" if what
                         else mpgemm_status_string(status))


def lib() -> ctypes.CDLL:
    """Load libmpgemm.so from this package directory (built in-tree)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is not built; run `python -m precision_dense_gemm_tiled_amd.build` "
                "(hipcc, gfx950)")
        L = ctypes.CDLL(lib_path)
        L.mpgemm_create.argtypes = [ctypes.POINTER(_vp), ctypes.c_int]
        L.mpgemm_create.restype = ctypes.c_int
        L.mpgemm_destroy.argtypes = [_vp]
        L.mpgemm_destroy.restype = ctypes.c_int
        L.mpgemm_status_string.argtypes = [ctypes.c_int]
        L.mpgemm_status_string.restype = ctypes.c_char_p
        for name in ("mpgemm_run_f16", "mpgemm_run_i8", "mpgemm_run_i4",
                     "mpgemm_run_f16_kn", "mpgemm_run_i8_kn", "mpgemm_run_i4_kn"):
            f = getattr(L, name)
            f.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
            f.restype = ctypes.c_int
        L.mpgemm_run_w4a16.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                       _vp, _i64, _i64, _vp, _i64, _vp]
        L.mpgemm_run_w4a16.restype = ctypes.c_int
        L.mpgemm_run_w4a16_noalloc.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                               _vp, _i64, _i64, _vp, _i64, _vp]
        L.mpgemm_run_w4a16_noalloc.restype = ctypes.c_int
        L.mpgemm_run_w4a4.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                      _vp, _i64, _vp]
        L.mpgemm_run_w4a4.restype = ctypes.c_int
        L.mpgemm_run_w4a4_lowrank.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                              _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
        L.mpgemm_run_w4a4_lowrank.restype = ctypes.c_int
        L.mpgemm_plan_gemm.argtypes = [ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.mpgemm_plan_gemm.restype = ctypes.c_int
        L.mpgemm_plan_w4a16.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i64)]
        L.mpgemm_plan_w4a16.restype = ctypes.c_int
        L.mpgemm_quantize_w4.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
        L.mpgemm_quantize_w4.restype = ctypes.c_int
        L.mpgemm_stream_read.argtypes = [_vp, _i64, ctypes.c_int, _vp, _i64, _vp]
        L.mpgemm_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ raw C-ABI

def mpgemm_status_string(status: int) -> str:
    return lib().mpgemm_status_string(int(status)).decode()


def mpgemm_create(device: int = -1) -> int:
    h = _vp()
    st = lib().mpgemm_create(ctypes.byref(h), int(device))
    if st != MPGEMM_OK:
        raise MpgemmError(st, "mpgemm_create")
    return h.value


def mpgemm_destroy(handle) -> int:
    return lib().mpgemm_destroy(handle)


def mpgemm_run_f16(h, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_f16(h, M, N, K, A, lda, B, ldb, C, ldc, stream)


def mpgemm_run_i8(h, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_i8(h, M, N, K, A, lda, B, ldb, C, ldc, stream)


def mpgemm_run_i4(h, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_i4(h, M, N, K, A, lda, B, ldb, C, ldc, stream)


def mpgemm_run_f16_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_f16_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream)


def mpgemm_run_i8_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_i8_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream)


def mpgemm_run_i4_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None) -> int:
    return lib().mpgemm_run_i4_kn(h, M, N, K, A, lda, Bt, ldbt, C, ldc, stream)


def mpgemm_run_w4a16(h, M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, stream=None) -> int:
    return lib().mpgemm_run_w4a16(h, M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, stream)


def mpgemm_run_w4a16_noalloc(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, stream=None) -> int:
    return lib().mpgemm_run_w4a16_noalloc(M, N, K, X, ldx, Wq, ldw, S, lds, group_size, Y, ldy, stream)


def mpgemm_run_w4a4(h, M, N, K, A, lda, B, ldb, SX, SW, bias, Y, ldy, stream=None) -> int:
    return lib().mpgemm_run_w4a4(h, M, N, K, A, lda, B, ldb, SX, SW, bias, Y, ldy, stream)


def mpgemm_run_w4a4_lowrank(h, M, N, K, A, lda, B, ldb, SX, SW, bias, X, ldx, LD, ldd, LU, ldu, R, Y, ldy,
                            stream=None) -> int:
    return lib().mpgemm_run_w4a4_lowrank(h, M, N, K, A, lda, B, ldb, SX, SW, bias, X, ldx, LD, ldd, LU, ldu, R,
                                         Y, ldy, stream)


def mpgemm_plan_gemm(precision, M, N, K, cu_count=256):
    """(status, tile configuration, stream-K grid (0: data-parallel), tiles run
    whole before the stream-K part) of a GEMM call; precision 0 f16, 1 i8,
    2 i4, 3 w4a4."""
    cfg, grid, tdp = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_int(-1)
    st = lib().mpgemm_plan_gemm(precision, M, N, K, cu_count, ctypes.byref(cfg), ctypes.byref(grid),
                                ctypes.byref(tdp))
    return st, cfg.value, grid.value, tdp.value


def mpgemm_plan_w4a16(M, N, K, cu_count=256):
    """(status, configuration, K splits, K per split) of a weight-only call."""
    cfg, ks, kslice = ctypes.c_int(-1), ctypes.c_int(0), ctypes.c_int64(0)
    st = lib().mpgemm_plan_w4a16(M, N, K, cu_count, ctypes.byref(cfg), ctypes.byref(ks), ctypes.byref(kslice))
    return st, cfg.value, ks.value, kslice.value


def mpgemm_quantize_w4(h, N, K, W, ldw, group_size, Wq, ldwq, S, lds, stream=None) -> int:
    return lib().mpgemm_quantize_w4(h, N, K, W, ldw, group_size, Wq, ldwq, S, lds, stream)


def mpgemm_stream_read(src, nbytes, loads_per_lane, sink, sink_words, stream=None) -> int:
    return lib().mpgemm_stream_read(src, nbytes, loads_per_lane, sink, sink_words, stream)


# ------------------------------------------------------------------ torch helpers

class Handle:
    """Owns one mpgemm handle (destroyed on close / garbage collection)."""

    def __init__(self, device: int = -1):
        self.value = mpgemm_create(device)

    def close(self):
        if self.value:
            mpgemm_destroy(self.value)
            self.value = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


_default = {}


def default_handle(device=None) -> int:
    import torch
    dev = torch.cuda.current_device() if device is None else int(device)
    if dev not in _default:
        _default[dev] = Handle(dev)
    return _default[dev].value


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _rows(t, dtype, name):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(1) == 1)")
    return t.stride(0) if t.size(0) > 1 else max(t.size(1), 1)


def _check(st, what):
    if st != MPGEMM_OK:
        raise MpgemmError(st, what)


def gemm_f16(A, B, out=None, handle=None, stream=None):
    """C = A @ B.T with fp16 A (M x K), B (N x K) -> fp32 C (M x N)."""
    import torch
    lda, ldb = _rows(A, torch.float16, "A"), _rows(B, torch.float16, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    C = torch.empty((M, N), dtype=torch.float32, device=A.device) if out is None else out
    ldc = _rows(C, torch.float32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_f16(h, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                          _stream(stream)), "mpgemm_run_f16")
    return C


def gemm_i8(A, B, out=None, handle=None, stream=None):
    """C = A @ B.T with int8 A (M x K), B (N x K) -> int32 C (M x N), exact."""
    import torch
    lda, ldb = _rows(A, torch.int8, "A"), _rows(B, torch.int8, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    C = torch.empty((M, N), dtype=torch.int32, device=A.device) if out is None else out
    ldc = _rows(C, torch.int32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_i8(h, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                         _stream(stream)), "mpgemm_run_i8")
    return C


def gemm_f16_kn(A, Bt, out=None, handle=None, stream=None):
    """C = A @ Bt with fp16 A (M x K), Bt (K x N, the transposed-B layout)
    -> fp32 C (M x N)."""
    import torch
    lda, ldbt = _rows(A, torch.float16, "A"), _rows(Bt, torch.float16, "Bt")
    M, K = A.shape
    if Bt.shape[0] != K:
        raise ValueError("A and Bt disagree on K")
    N = Bt.shape[1]
    C = torch.empty((M, N), dtype=torch.float32, device=A.device) if out is None else out
    ldc = _rows(C, torch.float32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_f16_kn(h, M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldbt, C.data_ptr(), ldc,
                             _stream(stream)), "mpgemm_run_f16_kn")
    return C


def gemm_i8_kn(A, Bt, out=None, handle=None, stream=None):
    """C = A @ Bt with int8 A (M x K), Bt (K x N) -> int32 C (M x N), exact."""
    import torch
    lda, ldbt = _rows(A, torch.int8, "A"), _rows(Bt, torch.int8, "Bt")
    M, K = A.shape
    if Bt.shape[0] != K:
        raise ValueError("A and Bt disagree on K")
    N = Bt.shape[1]
    C = torch.empty((M, N), dtype=torch.int32, device=A.device) if out is None else out
    ldc = _rows(C, torch.int32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_i8_kn(h, M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldbt, C.data_ptr(), ldc,
                            _stream(stream)), "mpgemm_run_i8_kn")
    return C


def gemm_i4_kn(A, Bt, N, out=None, handle=None, stream=None):
    """C = A @ Bt for signed INT4: A (M x K nibbles packed along K, uint8),
    Bt (K x N nibbles packed two per byte along n, low nibble = even n) ->
    int32 C (M x N), exact."""
    import torch
    lda_b, ldbt_b = _rows(A, torch.uint8, "A"), _rows(Bt, torch.uint8, "Bt")
    M, K = A.shape[0], Bt.shape[0]
    if 2 * Bt.shape[1] < N or 2 * A.shape[1] < K:
        raise ValueError("packed rows shorter than N or K")
    C = torch.empty((M, N), dtype=torch.int32, device=A.device) if out is None else out
    ldc = _rows(C, torch.int32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_i4_kn(h, M, N, K, A.data_ptr(), 2 * lda_b, Bt.data_ptr(), 2 * ldbt_b, C.data_ptr(),
                            ldc, _stream(stream)), "mpgemm_run_i4_kn")
    return C


def gemm_i4(A, B, K, out=None, handle=None, stream=None):
    """C = A @ B.T for packed signed INT4 rows (uint8 tensors, K nibbles per
    row, low nibble = even k) -> int32 C, exact."""
    import torch
    lda_b, ldb_b = _rows(A, torch.uint8, "A"), _rows(B, torch.uint8, "B")
    M, N = A.shape[0], B.shape[0]
    C = torch.empty((M, N), dtype=torch.int32, device=A.device) if out is None else out
    ldc = _rows(C, torch.int32, "C")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_i4(h, M, N, K, A.data_ptr(), 2 * lda_b, B.data_ptr(), 2 * ldb_b,
                         C.data_ptr(), ldc, _stream(stream)), "mpgemm_run_i4")
    return C


def gemm_w4a16(X, Wq, S, group_size, out=None, handle=None, stream=None):
    """Y = X @ dequant(Wq).T: fp16 X (M x K), packed INT4 Wq (N x K/2 uint8),
    fp16 scales S (N x K/G) -> fp16 Y (M x N)."""
    import torch
    ldx = _rows(X, torch.float16, "X")
    ldw_b = _rows(Wq, torch.uint8, "Wq")
    lds = _rows(S, torch.float16, "S")
    M, K = X.shape
    N = Wq.shape[0]
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    ldy = _rows(Y, torch.float16, "Y")
    h = default_handle(X.device.index) if handle is None else handle
    _check(mpgemm_run_w4a16(h, M, N, K, X.data_ptr(), ldx, Wq.data_ptr(), 2 * ldw_b,
                            S.data_ptr(), lds, group_size, Y.data_ptr(), ldy, _stream(stream)),
           "mpgemm_run_w4a16")
    return Y


def gemm_w4a16_noalloc(X, Wq, S, group_size, out=None, stream=None):
    """gemm_w4a16 through the allocation-free entry point (no handle; the
    current device's static scratch; `out` preallocated by the caller when
    nothing may be allocated)."""
    import torch
    ldx = _rows(X, torch.float16, "X")
    ldw_b = _rows(Wq, torch.uint8, "Wq")
    lds = _rows(S, torch.float16, "S")
    M, K = X.shape
    N = Wq.shape[0]
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    ldy = _rows(Y, torch.float16, "Y")
    _check(mpgemm_run_w4a16_noalloc(M, N, K, X.data_ptr(), ldx, Wq.data_ptr(), 2 * ldw_b,
                                    S.data_ptr(), lds, group_size, Y.data_ptr(), ldy, _stream(stream)),
           "mpgemm_run_w4a16_noalloc")
    return Y


def quantize_w4(W, group_size, out_q=None, out_s=None, handle=None, stream=None):
    """Symmetric per-(row, group) INT4 quantisation of fp16 weights W (N x K):
    returns packed Wq (N x K/2 uint8) and fp16 scales S (N x K/G), the inputs
    of gemm_w4a16."""
    import torch
    ldw = _rows(W, torch.float16, "W")
    N, K = W.shape
    Q = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device) if out_q is None else out_q
    S = (torch.empty((N, K // group_size if group_size > 0 else 0), dtype=torch.float16, device=W.device)
         if out_s is None else out_s)
    ldq_b = _rows(Q, torch.uint8, "Wq")
    lds = _rows(S, torch.float16, "S")
    h = default_handle(W.device.index) if handle is None else handle
    _check(mpgemm_quantize_w4(h, N, K, W.data_ptr(), ldw, group_size, Q.data_ptr(), 2 * ldq_b,
                              S.data_ptr(), lds, _stream(stream)), "mpgemm_quantize_w4")
    return Q, S


def gemm_w4a4(A, B, K, sx, sw, bias=None, out=None, handle=None, stream=None):
    """Y = fp16((A_int4 @ B_int4.T) * sx[:, None] * sw[None, :] + bias): packed
    INT4 A (M x K/2 uint8) and B (N x K/2 uint8), fp16 sx (M), sw (N), bias (N
    or None) -> fp16 Y (M x N)."""
    import torch
    lda_b = _rows(A, torch.uint8, "A")
    ldb_b = _rows(B, torch.uint8, "B")
    M, N = A.shape[0], B.shape[0]
    for name, v, n in (("sx", sx, M), ("sw", sw, N)) + ((("bias", bias, N),) if bias is not None else ()):
        if v.dtype != torch.float16 or v.numel() != n or not v.is_contiguous() or not v.is_cuda:
            raise ValueError(f"{name}: expected {n} contiguous fp16 values on the device")
    Y = torch.empty((M, N), dtype=torch.float16, device=A.device) if out is None else out
    ldy = _rows(Y, torch.float16, "Y")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_w4a4(h, M, N, K, A.data_ptr(), 2 * lda_b, B.data_ptr(), 2 * ldb_b, sx.data_ptr(),
                           sw.data_ptr(), bias.data_ptr() if bias is not None else None, Y.data_ptr(), ldy,
                           _stream(stream)), "mpgemm_run_w4a4")
    return Y


def gemm_w4a4_lowrank(A, B, K, sx, sw, X, LD, LU, bias=None, out=None, handle=None, stream=None):
    """gemm_w4a4 plus the low-rank branch: Y = fp16(((A_int4 @ B_int4.T) *
    sx[:, None] * sw[None, :] + fp16(X @ LD.T) @ LU.T) + bias), with fp16 X
    (M x K, the unquantised activations), LD (R x K) and LU (N x R)."""
    import torch
    lda_b = _rows(A, torch.uint8, "A")
    ldb_b = _rows(B, torch.uint8, "B")
    ldx = _rows(X, torch.float16, "X")
    ldd = _rows(LD, torch.float16, "LD")
    ldu = _rows(LU, torch.float16, "LU")
    M, N, R = A.shape[0], B.shape[0], LD.shape[0]
    if X.shape != (M, K) or LD.shape[1] != K or LU.shape != (N, R):
        raise ValueError(f"shapes: X {tuple(X.shape)}, LD {tuple(LD.shape)}, LU {tuple(LU.shape)} for "
                         f"M = {M}, N = {N}, K = {K}")
    for name, v, n in (("sx", sx, M), ("sw", sw, N)) + ((("bias", bias, N),) if bias is not None else ()):
        if v.dtype != torch.float16 or v.numel() != n or not v.is_contiguous() or not v.is_cuda:
            raise ValueError(f"{name}: expected {n} contiguous fp16 values on the device")
    Y = torch.empty((M, N), dtype=torch.float16, device=A.device) if out is None else out
    ldy = _rows(Y, torch.float16, "Y")
    h = default_handle(A.device.index) if handle is None else handle
    _check(mpgemm_run_w4a4_lowrank(h, M, N, K, A.data_ptr(), 2 * lda_b, B.data_ptr(), 2 * ldb_b, sx.data_ptr(),
                                   sw.data_ptr(), bias.data_ptr() if bias is not None else None, X.data_ptr(),
                                   ldx, LD.data_ptr(), ldd, LU.data_ptr(), ldu, R, Y.data_ptr(), ldy,
                                   _stream(stream)), "mpgemm_run_w4a4_lowrank")
    return Y
