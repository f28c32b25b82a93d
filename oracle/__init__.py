"""ctypes front end of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__.py and the
cpu_baseline leg of bench.py use it. The GPU library never imports it.

Every function takes and returns numpy arrays; the arithmetic happens in
oracle.c (see oracle.h for the pages each definition follows).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MPGEMM_ORACLE_LIB points the pins at another build of oracle.c (the
# mutation test's deliberately broken copies); unset, the library built here.
_LIB_PATH = os.environ.get("MPGEMM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_OVERFLOW = 0, 1, 2

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} missing: run python oracle/build.py")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_f16_decode.restype = ctypes.c_double
        L.oracle_f16_encode_rne.argtypes = [ctypes.c_double]
        L.oracle_f16_encode_rne.restype = ctypes.c_uint16
        L.oracle_i4_get.argtypes = [_p, _i64]
        L.oracle_i4_get.restype = ctypes.c_int
        for name in ("oracle_gemm_i8", "oracle_gemm_i4", "oracle_gemm_f16"):
            f = getattr(L, name)
            f.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]
            f.restype = ctypes.c_int
        L.oracle_gemm_w4a16.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64,
                                        _p, _i64, _i64, _p, _i64, _p, _i64]
        L.oracle_gemm_w4a16.restype = ctypes.c_int
        L.oracle_gemm_w4a4.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _p, _i64]
        L.oracle_gemm_w4a4.restype = ctypes.c_int
        L.oracle_w4a4_lowrank.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64]
        L.oracle_w4a4_lowrank.restype = ctypes.c_int
        L.oracle_quantize_w4.argtypes = [_i64, _i64, _p, _i64, _i64, _p, _i64, _p, _i64]
        L.oracle_quantize_w4.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _rows(a, dtype):
    a = np.asarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.ndim == 2, "2-D row-major array required"
    if a.shape[1] > 1 and a.strides[1] != a.itemsize:
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1]
    return a, max(ld, a.shape[1])


def threads() -> int:
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the following oracle calls (timing only)."""
    lib().oracle_set_threads(int(n))


def f16_decode(bits: int) -> float:
    return lib().oracle_f16_decode(int(bits) & 0xFFFF)


def f16_encode_rne(x: float) -> int:
    return int(lib().oracle_f16_encode_rne(float(x)))


def f16_encode_rne_array(x) -> np.ndarray:
    enc = lib().oracle_f16_encode_rne
    x = np.asarray(x, dtype=np.float64)
    return np.array([enc(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def i4_get(row: np.ndarray, k: int) -> int:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return lib().oracle_i4_get(_ptr(row), int(k))


def gemm_i8(A, B, check=True):
    """C = A * B^T exactly; A is M x K int8, B is N x K int8 -> M x N int32."""
    A, lda = _rows(A, np.int8)
    B, ldb = _rows(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    C = np.zeros((M, N), dtype=np.int32)
    st = lib().oracle_gemm_i8(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), N)
    if check and st != OK:
        raise ValueError(f"oracle_gemm_i8 status {st}")
    return C


def gemm_i4(Ap, Bp, K, check=True):
    """C = A * B^T for packed signed INT4 rows (K nibbles per row, K even)."""
    Ap, lda_b = _rows(Ap, np.uint8)
    Bp, ldb_b = _rows(Bp, np.uint8)
    M, N = Ap.shape[0], Bp.shape[0]
    assert Ap.shape[1] * 2 >= K and Bp.shape[1] * 2 >= K
    C = np.zeros((M, N), dtype=np.int32)
    st = lib().oracle_gemm_i4(M, N, K, _ptr(Ap), 2 * lda_b, _ptr(Bp), 2 * ldb_b, _ptr(C), N)
    if check and st != OK:
        raise ValueError(f"oracle_gemm_i4 status {st}")
    return C


def gemm_f16(A, B):
    """C = A * B^T in double; A, B are binary16 bit arrays (uint16) or float16."""
    A = np.asarray(A)
    B = np.asarray(B)
    if A.dtype == np.float16:
        A = A.view(np.uint16)
    if B.dtype == np.float16:
        B = B.view(np.uint16)
    A, lda = _rows(A, np.uint16)
    B, ldb = _rows(B, np.uint16)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    C = np.zeros((M, N), dtype=np.float64)
    st = lib().oracle_gemm_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), N)
    if st != OK:
        raise ValueError(f"oracle_gemm_f16 status {st}")
    return C


def gemm_w4a16(X, Wp, S, K, G, want_t2=False):
    """Y = sum_k x q s (double, unrounded); optionally also T2 = sum_k (x q s)^2."""
    X = np.asarray(X)
    S = np.asarray(S)
    if X.dtype == np.float16:
        X = X.view(np.uint16)
    if S.dtype == np.float16:
        S = S.view(np.uint16)
    X, ldx = _rows(X, np.uint16)
    Wp, ldw_b = _rows(Wp, np.uint8)
    S, lds = _rows(S, np.uint16)
    M, N = X.shape[0], Wp.shape[0]
    Y = np.zeros((M, N), dtype=np.float64)
    T2 = np.zeros((M, N), dtype=np.float64) if want_t2 else None
    st = lib().oracle_gemm_w4a16(M, N, K, _ptr(X), ldx, _ptr(Wp), 2 * ldw_b,
                                 _ptr(S), lds, G, _ptr(Y), N, _ptr(T2), N)
    if st != OK:
        raise ValueError(f"oracle_gemm_w4a16 status {st}")
    return (Y, T2) if want_t2 else Y


def quantize_w4(W, G):
    """Symmetric per-(row, group) INT4 quantisation of fp16 weights W (N x K):
    returns (packed Q as N x K/2 uint8, scales S as N x K/G float16)."""
    W = np.asarray(W)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    W, ldw = _rows(W, np.uint16)
    N, K = W.shape
    Q = np.zeros((N, (K + 1) // 2), dtype=np.uint8)
    S = np.zeros((N, K // G if G > 0 else 0), dtype=np.uint16)
    st = lib().oracle_quantize_w4(N, K, _ptr(W), ldw, G, _ptr(Q), 2 * Q.shape[1], _ptr(S), max(S.shape[1], 1))
    if st != OK:
        raise ValueError(f"oracle_quantize_w4 status {st}")
    return Q, S.view(np.float16)


def gemm_w4a4(Ap, Bp, K, SX, SW, BIAS=None):
    """Y = (sum_k qa qb) * SX[m] * SW[n] + BIAS[n] (double, unrounded)."""
    def bits(v):
        v = np.ascontiguousarray(np.asarray(v))
        return v.view(np.uint16) if v.dtype == np.float16 else v.astype(np.uint16)
    Ap, lda_b = _rows(Ap, np.uint8)
    Bp, ldb_b = _rows(Bp, np.uint8)
    M, N = Ap.shape[0], Bp.shape[0]
    sx, sw = bits(SX), bits(SW)
    b = bits(BIAS) if BIAS is not None else None
    Y = np.zeros((M, N), dtype=np.float64)
    st = lib().oracle_gemm_w4a4(M, N, K, _ptr(Ap), 2 * lda_b, _ptr(Bp), 2 * ldb_b,
                                _ptr(sx), _ptr(sw), _ptr(b) if b is not None else None, _ptr(Y), N)
    if st != OK:
        raise ValueError(f"oracle_gemm_w4a4 status {st}")
    return Y


def w4a4_lowrank(X, LD, LU):
    """The low-rank branch of the W4A4 formula: U = X LD^T (M x R, double) and
    L = binary16_rne(U) LU^T (M x N, double, unrounded), for fp16 X (M x K),
    LD (R x K) and LU (N x R). Returns (U, L)."""
    def bits(v):
        v = np.asarray(v)
        return v.view(np.uint16) if v.dtype == np.float16 else v
    X, ldx = _rows(bits(X), np.uint16)
    LD, ldd = _rows(bits(LD), np.uint16)
    LU, ldu = _rows(bits(LU), np.uint16)
    M, K = X.shape
    R, N = LD.shape[0], LU.shape[0]
    assert LD.shape[1] == K and LU.shape[1] == R, "shapes"
    U = np.zeros((M, R), dtype=np.float64)
    L = np.zeros((M, N), dtype=np.float64)
    st = lib().oracle_w4a4_lowrank(M, N, K, R, _ptr(X), ldx, _ptr(LD), ldd, _ptr(LU), ldu,
                                   _ptr(U), max(R, 1), _ptr(L), max(N, 1))
    if st != OK:
        raise ValueError(f"oracle_w4a4_lowrank status {st}")
    return U, L
