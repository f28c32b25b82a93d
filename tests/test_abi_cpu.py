"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/mpgemm.h declares, and reports argument errors before any device
work (the handle is checked last, so a NULL handle reaches every check)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpgemm.h")


@pytest.fixture(scope="module")
def mp():
    import precision_dense_gemm_tiled_amd as mp
    if not os.path.exists(mp.lib_path):
        from precision_dense_gemm_tiled_amd import build
        build.build()
    mp.lib()
    return mp


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpgemm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_symbols()
    for n in ["mpgemm_create", "mpgemm_destroy", "mpgemm_status_string", "mpgemm_run_f16",
              "mpgemm_run_i8", "mpgemm_run_i4", "mpgemm_run_w4a16", "mpgemm_run_w4a4", "mpgemm_quantize_w4",
              "mpgemm_run_w4a4_lowrank", "mpgemm_run_f16_kn", "mpgemm_run_i8_kn", "mpgemm_run_i4_kn"]:
        assert n in names


def test_library_exports_every_declared_symbol(mp):
    L = mp.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_status_strings(mp):
    assert mp.mpgemm_status_string(0) == "MPGEMM_OK"
    assert mp.mpgemm_status_string(2) == "MPGEMM_ERR_UNSUPPORTED"
    assert mp.mpgemm_status_string(3) == "MPGEMM_ERR_DEVICE"
    assert mp.mpgemm_status_string(99) == "MPGEMM_UNKNOWN_STATUS"


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_create_without_gpu_reports_device_error(mp):
    h = ctypes.c_void_p()
    assert mp.lib().mpgemm_create(ctypes.byref(h), -1) == mp.MPGEMM_ERR_DEVICE
    assert h.value is None
    with pytest.raises(mp.MpgemmError):
        mp.mpgemm_create()


def test_destroy_null_is_ok(mp):
    assert mp.mpgemm_destroy(None) == 0
    assert mp.lib().mpgemm_create(None, 0) == mp.MPGEMM_ERR_INVALID_ARG


# fake, never dereferenced device addresses (16-byte aligned)
A, B, C, S = 0x10000, 0x20000, 0x30000, 0x40000


@pytest.mark.parametrize("call,expect", [
    # sizes
    (("i8", -1, 4, 4, A, 16, B, 16, C, 16), 1),
    (("i8", 4, 4, -2, A, 16, B, 16, C, 16), 1),
    # zero-sized problems are no-ops
    (("i8", 0, 4, 4, 0, 16, 0, 16, 0, 16), 0),
    (("f16", 4, 0, 4, 0, 16, 0, 16, 0, 16), 0),
    # pointers
    (("i8", 4, 4, 16, 0, 16, B, 16, C, 16), 1),
    (("i8", 4, 4, 16, A, 16, B, 16, 0, 16), 1),
    # leading dimensions
    (("i8", 4, 4, 32, A, 16, B, 32, C, 16), 1),
    (("f16", 4, 8, 16, A, 16, B, 16, C, 4), 1),
    # unaligned operands are accepted (byte-gather kernel); C needs 4 bytes
    (("i8", 4, 4, 16, A + 4, 16, B, 16, C, 16), 1),
    (("i8", 4, 4, 16, A, 24, B, 16, C, 16), 1),
    (("f16", 4, 4, 16, A, 20, B, 16, C, 16), 1),
    (("f16", 4, 6, 16, A, 16, B, 16, C, 6), 1),
    (("f16", 4, 4, 16, A, 16, B, 16, C + 2, 16), 2),
    (("i8", 4, 4, 16, A, 16, B, 16, C + 1, 16), 2),
    # INT4: odd K or odd ld
    (("i4", 4, 4, 31, A, 32, B, 32, C, 16), 2),
    (("i4", 4, 4, 32, A, 33, B, 32, C, 16), 2),
    # integer K bound (exact int32 results)
    (("i8", 4, 4, 131072, A, 131072, B, 131072, C, 16), 2),
    (("i4", 4, 4, 131072, A, 131072, B, 131072, C, 16), 2),
    # everything valid: only the NULL handle is left to report
    (("i8", 4, 4, 16, A, 16, B, 16, C, 16), 1),
])
def test_gemm_argument_errors_without_device(mp, call, expect):
    prec, *args = call
    f = {"i8": mp.mpgemm_run_i8, "i4": mp.mpgemm_run_i4, "f16": mp.mpgemm_run_f16}[prec]
    assert f(None, *args, None) == expect


@pytest.mark.parametrize("call,expect", [
    # sizes, no-ops, pointers
    (("i8", -1, 16, 16, A, 16, B, 16, C, 16), 1),
    (("i8", 0, 16, 16, 0, 16, 0, 16, 0, 16), 0),
    (("f16", 4, 16, 16, A, 16, 0, 16, C, 16), 1),
    # Bt is K x N: its leading dimension is checked against N, not K
    (("i8", 4, 32, 16, A, 16, B, 16, C, 32), 1),
    (("i8", 4, 16, 32, A, 32, B, 16, C, 16), 1),      # ldbt = N < K is fine: NULL handle left
    (("f16", 4, 16, 16, A, 8, B, 16, C, 16), 1),      # lda < K
    # one kernel only: 16-byte rows and bases, else unsupported
    (("i8", 4, 16, 16, A, 16, B + 8, 16, C, 16), 2),
    (("i8", 4, 16, 16, A, 24, B, 16, C, 16), 2),
    (("f16", 4, 12, 16, A, 16, B, 12, C, 12), 2),     # Bt rows of 24 bytes
    (("f16", 4, 16, 16, A, 16, B, 16, C + 2, 16), 2),
    # INT4: K, lda, ldbt even; Bt rows of ldbt / 2 bytes, a multiple of 16
    (("i4", 4, 32, 31, A, 32, B, 32, C, 32), 2),
    (("i4", 4, 31, 32, A, 32, B, 33, C, 32), 2),
    (("i4", 4, 31, 32, A, 32, B, 48, C, 32), 2),
    (("i4", 4, 31, 32, A, 32, B, 32, C, 32), 1),      # odd N: NULL handle left
    # integer K bound
    (("i8", 4, 16, 131072, A, 131072, B, 16, C, 16), 2),
])
def test_gemm_kn_argument_errors_without_device(mp, call, expect):
    prec, *args = call
    f = {"i8": mp.mpgemm_run_i8_kn, "i4": mp.mpgemm_run_i4_kn, "f16": mp.mpgemm_run_f16_kn}[prec]
    assert f(None, *args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((1, 16, 256, A, 256, B, 256, S, 2, 128, C, 16), 1),     # valid: NULL handle
    ((1, 16, 256, A, 256, B, 256, S, 2, 100, C, 16), 2),     # G not a power of two
    ((1, 16, 256, A, 256, B, 256, S, 16, 16, C, 16), 2),     # G below 32
    ((1, 16, 192, A, 256, B, 256, S, 2, 128, C, 16), 2),     # K % G != 0
    ((1, 16, 256, A, 256, B, 256, S, 1, 128, C, 16), 1),     # lds < K/G
    ((1, 16, 256, A, 256, B, 256, S + 1, 2, 128, C, 16), 2),  # scales not 2-byte aligned
    ((1, 16, 256, A, 256, B, 250, S, 2, 128, C, 16), 1),     # ldw < K
    ((1, 16, 256, A, 260, B, 256, S, 2, 128, C, 16), 2),     # X row stride not 16 B
    ((1, 16, 256, A + 2, 256, B, 256, S, 2, 128, C, 16), 2),  # X not 16-byte aligned
    ((1, 16, 256, A, 256, B, 256, S, 2, 128, C + 1, 16), 2),  # Y not 2-byte aligned
    ((1, 10, 256, A, 256, B, 256, S, 2, 128, C + 2, 10), 1),  # any Y stride: NULL handle left
    ((0, 16, 256, 0, 256, 0, 256, 0, 2, 128, 0, 16), 0),     # M = 0: no-op
])
def test_w4a16_argument_errors_without_device(mp, args, expect):
    assert mp.mpgemm_run_w4a16(None, *args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((1, 16, 256, A, 256, B, 256, S, 2, 100, C, 16), 2),     # G not a power of two
    ((1, 16, 192, A, 256, B, 256, S, 2, 128, C, 16), 2),     # K % G != 0
    ((1, 16, 256, A, 256, B, 256, S, 1, 128, C, 16), 1),     # lds < K/G
    ((1, 16, 256, A, 256, B, 250, S, 2, 128, C, 16), 1),     # ldw < K
    ((1, 16, 256, A + 2, 256, B, 256, S, 2, 128, C, 16), 2),  # X not 16-byte aligned
    ((1, 16, 256, A, 256, B, 256, S, 2, 128, C + 1, 16), 2),  # Y not 2-byte aligned
    ((-1, 16, 256, A, 256, B, 256, S, 2, 128, C, 16), 1),    # negative size
    ((1, 16, 256, 0, 256, B, 256, S, 2, 128, C, 16), 1),     # NULL activations
    ((0, 16, 256, 0, 256, 0, 256, 0, 2, 128, 0, 16), 0),     # M = 0: no-op
])
def test_w4a16_noalloc_argument_errors_without_device(mp, args, expect):
    """The allocation-free entry point makes the same argument checks as
    mpgemm_run_w4a16, before any HIP call."""
    assert mp.mpgemm_run_w4a16_noalloc(*args, None) == expect


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_w4a16_noalloc_without_gpu_reports_device_error(mp):
    """With valid arguments and no GPU, the device query fails first."""
    args = (1, 16, 256, A, 256, B, 256, S, 2, 128, C, 16)
    assert mp.mpgemm_run_w4a16_noalloc(*args, None) == mp.MPGEMM_ERR_DEVICE


@pytest.mark.parametrize("args,expect", [
    ((16, 256, A, 256, 128, B, 256, S, 2), 1),       # valid: NULL handle left
    ((-1, 256, A, 256, 128, B, 256, S, 2), 1),      # negative size
    ((0, 256, 0, 256, 128, 0, 256, 0, 2), 0),       # N = 0: no-op
    ((16, 0, 0, 0, 128, 0, 0, 0, 0), 0),            # K = 0: no-op
    ((16, 256, A, 256, 100, B, 256, S, 2), 2),      # G not a power of two
    ((16, 256, A, 256, 16, B, 256, S, 16), 2),      # G below 32
    ((16, 2048, A, 2048, 1024, B, 2048, S, 2), 2),  # G above 512
    ((16, 192, A, 192, 128, B, 192, S, 2), 2),      # K % G != 0
    ((16, 256, A, 200, 128, B, 256, S, 2), 1),      # ldw < K
    ((16, 256, A, 256, 128, B, 256, S, 1), 1),      # lds < K / G
    ((16, 256, A + 2, 256, 128, B, 256, S, 2), 2),  # W not 16-byte aligned
    ((16, 256, A, 260, 128, B, 256, S, 2), 2),      # W row stride not 16 bytes
    ((16, 256, A, 256, 128, B + 2, 256, S, 2), 2),  # Wq not 4-byte aligned
    ((16, 256, A, 256, 128, B, 258, S, 2), 2),      # Wq row stride not 4 bytes
    ((16, 256, A, 256, 128, B, 256, S + 1, 2), 2),  # S not 2-byte aligned
    ((16, 256, 0, 256, 128, B, 256, S, 2), 1),      # NULL weights
])
def test_quantize_argument_errors_without_device(mp, args, expect):
    assert mp.mpgemm_quantize_w4(None, *args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((4, 4, 32, A, 32, B, 32, S, S + 64, S + 128, C, 16), 1),      # valid: NULL handle left
    ((4, 4, 32, A, 32, B, 32, S, S + 64, 0, C, 16), 1),            # no bias is fine
    ((0, 4, 32, 0, 32, 0, 32, 0, 0, 0, 0, 16), 0),                 # M = 0: no-op
    ((4, 4, 31, A, 32, B, 32, S, S + 64, 0, C, 16), 2),            # odd K
    ((4, 4, 32, A, 33, B, 32, S, S + 64, 0, C, 16), 2),            # odd lda
    ((4, 4, 32, A, 32, B, 32, 0, S + 64, 0, C, 16), 1),            # no SX
    ((4, 4, 32, A, 32, B, 32, S, 0, 0, C, 16), 1),                 # no SW
    ((4, 4, 32, A, 32, B, 32, S + 1, S + 64, 0, C, 16), 2),        # SX not 2-byte aligned
    ((4, 4, 32, A, 32, B, 32, S, S + 64, S + 129, C, 16), 2),      # bias not 2-byte aligned
    ((4, 4, 32, A, 32, B, 32, S, S + 64, 0, C + 1, 16), 2),        # Y not 2-byte aligned
    ((4, 8, 32, A, 32, B, 32, S, S + 64, 0, C, 4), 1),             # ldy < N
    ((4, 4, 131072, A, 131072, B, 131072, S, S + 64, 0, C, 16), 2),  # K bound
])
def test_w4a4_argument_errors_without_device(mp, args, expect):
    assert mp.mpgemm_run_w4a4(None, *args, None) == expect


# (M, N, K, A, lda, B, ldb, SX, SW, bias, X, ldx, LD, ldd, LU, ldu, R, Y, ldy)
_LR = (4, 4, 32, A, 32, B, 32, S, S + 64, 0, A + 4096, 32, A + 8192, 32, A + 16384, 16, 16, C, 16)


def _lr(**kw):
    names = ["M", "N", "K", "A", "lda", "B", "ldb", "SX", "SW", "bias", "X", "ldx", "LD", "ldd", "LU", "ldu",
             "R", "Y", "ldy"]
    v = dict(zip(names, _LR))
    v.update(kw)
    return tuple(v[n] for n in names)


@pytest.mark.parametrize("args,expect", [
    (_lr(), 1),                                 # valid: NULL handle left
    (_lr(R=0), 1),                              # R = 0 is the plain W4A4 call (NULL handle left)
    (_lr(M=0), 0),                              # M = 0: no-op
    (_lr(R=-16), 1),                            # negative rank
    (_lr(R=24, ldu=24), 2),                     # rank not a multiple of 16
    (_lr(R=272, ldu=272), 2),                   # rank above MPGEMM_MAX_LOWRANK
    (_lr(LU=A + 16384 + 8), 2),                 # LU not 16-byte aligned
    (_lr(ldu=20, R=16), 2),                     # LU row stride not a multiple of 8
    (_lr(ldu=8), 1),                            # ldu < R
    (_lr(ldx=16), 1),                           # ldx < K
    (_lr(ldd=16), 1),                           # ldd < K
    (_lr(X=0), 1),                              # no X
    (_lr(LD=0), 1),                             # no down-projection
    (_lr(LU=0), 1),                             # no up-projection
    (_lr(X=A + 4097), 2),                       # X not 2-byte aligned
    (_lr(K=31), 2),                             # odd K (the W4A4 rule)
    (_lr(SX=0), 1),                             # no SX
])
def test_w4a4_lowrank_argument_errors_without_device(mp, args, expect):
    assert mp.mpgemm_run_w4a4_lowrank(None, *args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, 4096, 3, C, 4), 2),        # loads per lane not 1, 2, 4 or 8
    ((A, 4008, 1, C, 4), 2),        # not a multiple of 16 bytes
    ((A + 8, 4096, 1, C, 4), 2),    # source not 16-byte aligned
    ((A, 4096 * 8, 1, C, 4), 1),    # more workgroups than sink words
    ((0, 4096, 1, C, 4), 1),        # NULL source
    ((A, 4096, 1, 0, 4), 1),        # NULL sink
    ((A, -16, 1, C, 4), 1),         # negative size
])
def test_stream_read_argument_errors_without_device(mp, args, expect):
    assert mp.mpgemm_stream_read(*args, None) == expect
