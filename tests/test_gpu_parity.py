"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Integer paths must match bit for bit; FP16 within 2^-10 * sqrt(K) per element
(fp32 output against the fp64 oracle); W4A16 within the bar in gpu_util.
Every test compares every element of its output with the oracle, except the
W4A4 GEMM at 8192, which compares two full rows of every 256-row band of
output tiles.
"""
import numpy as np
import pytest

import oracle
import precision_dense_gemm_tiled_amd as mp
from precision_dense_gemm_tiled_amd import inputs
from tests.gpu_util import (B_DIRECT_CFGS, N_TILE_CFGS, PINGPONG_CFG, band_rows, dev, f16_tol, freivalds_int, host,
                            pack_i4, require_gpu, unpack_i4, w4a4_tol, w4a16_tol)

pytestmark = pytest.mark.gpu

SMALL_SHAPES = [(1, 1, 2), (1, 1, 64), (2, 3, 16), (7, 13, 34), (64, 64, 64), (100, 200, 300),
                (256, 256, 512), (257, 129, 1000), (513, 300, 64), (33, 700, 130), (1, 517, 258)]


@pytest.fixture(scope="module", autouse=True)
def gpu(oracle_lib):
    require_gpu()
    return True


def _run(prec, A, B, K):
    if prec == "i8":
        return host(mp.gemm_i8(dev(A), dev(B)))
    if prec == "i4":
        return host(mp.gemm_i4(dev(A), dev(B), K))
    return host(mp.gemm_f16(dev(A), dev(B)))


def _ref(prec, A, B, K):
    if prec == "i8":
        return oracle.gemm_i8(A, B)
    if prec == "i4":
        return oracle.gemm_i4(A, B, K)
    return oracle.gemm_f16(A, B)


def _compare(prec, got, ref, K, what):
    if prec == "f16":
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= f16_tol(K)), f"{what}: max err {err.max()} > {f16_tol(K)}"
    else:
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first {bad[:4].tolist()}"


# ------------------------------------------------------------------ small shapes

@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_small_shapes(prec, M, N, K):
    A, B = inputs.gemm_problem(prec, M, N, K, seed=M * 131 + N * 7 + K)
    got = _run(prec, A, B, K)
    _compare(prec, got, _ref(prec, A, B, K), K, f"{prec} {M}x{N}x{K}")


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
def test_every_tile_config(prec, monkeypatch):
    """Each tile configuration (forced through the ablation override) on a
    ragged shape spanning several tiles."""
    M, N, K = 300, 520, 200
    A, B = inputs.gemm_problem(prec, M, N, K, seed=77)
    ref = _ref(prec, A, B, K)
    for cfg in range(N_TILE_CFGS):
        monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        with mp.Handle() as h:
            a, b = dev(A), dev(B)
            if prec == "i8":
                got = host(mp.gemm_i8(a, b, handle=h.value))
            elif prec == "i4":
                got = host(mp.gemm_i4(a, b, K, handle=h.value))
            else:
                got = host(mp.gemm_f16(a, b, handle=h.value))
        _compare(prec, got, ref, K, f"{prec} cfg {cfg}")


# (M, N, K bytes per row): the ping-pong and B-direct kernels need K in whole
# 128-byte stages (ping-pong: at least two); ragged M and N tiles, a single
# output, one tile, a grid of several tiles with a longer K.
PINGPONG_SHAPES = [(300, 520, 256), (513, 260, 1024), (1, 1, 256), (256, 256, 384), (700, 1000, 2048)]
WHOLE_STAGE_CASES = ([(PINGPONG_CFG, *s) for s in PINGPONG_SHAPES] +
                     [(c, *s) for c in B_DIRECT_CFGS for s in PINGPONG_SHAPES + [(260, 300, 128)]])


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("cfg,M,N,kb", WHOLE_STAGE_CASES)
def test_whole_stage_config(prec, cfg, M, N, kb, monkeypatch):
    """The kernels that run only on K in whole 128-byte stages (the 256 x 256
    ping-pong kernel, the kernels that load B straight into registers),
    forced, against the oracle, and a second call on the same inputs
    bit-identical to the first."""
    K = {"i8": kb, "f16": kb // 2, "i4": 2 * kb}[prec]
    A, B = inputs.gemm_problem(prec, M, N, K, seed=1000 + M + N + kb)
    monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
    with mp.Handle() as h:
        a, b = dev(A), dev(B)
        runs = []
        for _ in range(2):
            if prec == "i8":
                runs.append(host(mp.gemm_i8(a, b, handle=h.value)))
            elif prec == "i4":
                runs.append(host(mp.gemm_i4(a, b, K, handle=h.value)))
            else:
                runs.append(host(mp.gemm_f16(a, b, handle=h.value)))
    _compare(prec, runs[0], _ref(prec, A, B, K), K, f"{prec} cfg {cfg} {M}x{N}x{K}")
    assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32)), "repeat differs"


# Transposed-B layout (B stored K x N), the control of the B-layout ablation:
# ragged M and N tiles with a K tail inside a stage, exactly one stage,
# several stages, a single output row, odd N (INT4 packs two n per byte),
# K = 0 (C = 0).
KN_SHAPES = [(300, 520, 200), (256, 256, 256), (513, 260, 1024), (1, 40, 64), (33, 47, 64), (70, 90, 0)]


def _padded_rows(a):
    """2-D host array -> device view of the same values whose rows start on
    16-byte boundaries (row stride padded with zeros)."""
    rows, width = a.shape
    pad = -(-max(width * a.itemsize, 1) // 16) * 16 // a.itemsize
    buf = np.zeros((max(rows, 2), pad), dtype=a.dtype)
    buf[:rows, :width] = a
    return dev(buf)[:rows, :width]


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("M,N,K", KN_SHAPES)
def test_transposed_b_layout(prec, M, N, K):
    """mpgemm_run_*_kn against the oracle of the usual N x K layout on the
    same values: Bt is B transposed (INT4: repacked two n per byte)."""
    if prec == "i4" and K % 2:
        pytest.skip("INT4 K is even")
    A, B = inputs.gemm_problem(prec, M, N, K, seed=5000 + M + N + K)
    ref = _ref(prec, A, B, K)
    if prec == "i4":
        vals = unpack_i4(B, K).T                     # K x N values
        if N % 2:
            vals = np.concatenate([vals, np.zeros((K, 1), dtype=vals.dtype)], axis=1)
        bt = pack_i4(vals) if K else np.zeros((0, (N + 1) // 2), dtype=np.uint8)
        got = host(mp.gemm_i4_kn(_padded_rows(A), _padded_rows(bt), N))
    else:
        bt = np.ascontiguousarray(B.T)
        f = mp.gemm_i8_kn if prec == "i8" else mp.gemm_f16_kn
        got = host(f(_padded_rows(A), _padded_rows(bt)))
    assert got.shape == (M, N)
    _compare(prec, got, ref, max(K, 1), f"{prec} kn {M}x{N}x{K}")


def test_i4_equals_i8_of_unpacked_on_gpu():
    M, N, K = 190, 260, 384
    Ap, Bp = inputs.gemm_problem("i4", M, N, K, seed=4242)
    c4 = _run("i4", Ap, Bp, K)
    c8 = _run("i8", unpack_i4(Ap, K), unpack_i4(Bp, K), K)
    assert np.array_equal(c4, c8)


def test_i4_extremes():
    K = 4096
    m8 = pack_i4(np.full((40, K), -8))
    p7 = pack_i4(np.full((70, K), 7))
    assert np.all(_run("i4", m8, m8, K) == 64 * K)
    assert np.all(_run("i4", m8, p7, K) == -56 * K)


def test_i8_extremes():
    K = 8192
    full = np.full((64, K), -128, dtype=np.int8)
    assert np.all(_run("i8", full, full, K) == 16384 * K)
    top = np.full((64, K), 127, dtype=np.int8)
    assert np.all(_run("i8", full, top, K) == -128 * 127 * K)


@pytest.mark.parametrize("streamk", ["0", "auto"])
def test_integer_k_bound(streamk, monkeypatch):
    """The largest K the integer calls accept: INT8 at K = 131071 (all -128:
    every sum 16384 K = 2^31 - 16384; K tail of 127 bytes) and INT4 at
    K = 131070 (all -8: the widened operands sum 256 * 64 K = 2^31 - 32768
    inside the kernel before the shift), plus random values against the
    oracle; data-parallel and with the default plan (which splits these long
    K loops over the grid)."""
    if streamk == "0":
        monkeypatch.setenv("MPGEMM_STREAMK", "0")
    with mp.Handle() as h:
        K = 131071
        m128 = np.full((40, K), -128, dtype=np.int8)
        c = host(mp.gemm_i8(dev(m128), dev(m128), handle=h.value))
        assert np.all(c == 16384 * K) and 16384 * K < 2 ** 31
        A, B = inputs.gemm_problem("i8", 33, 70, K, seed=131071)
        assert np.array_equal(host(mp.gemm_i8(dev(A), dev(B), handle=h.value)), oracle.gemm_i8(A, B))
        K = 131070
        m8 = pack_i4(np.full((40, K), -8))
        c = host(mp.gemm_i4(dev(m8), dev(m8), K, handle=h.value))
        assert np.all(c == 64 * K) and 256 * 64 * K < 2 ** 31
        A, B = inputs.gemm_problem("i4", 33, 70, K, seed=131070)
        assert np.array_equal(host(mp.gemm_i4(dev(A), dev(B), K, handle=h.value)), oracle.gemm_i4(A, B, K))


def test_f16_small_integers_bit_exact():
    """Integers in [-4, 4]: every partial sum is an integer below 2^24, so an
    fp32 accumulator is exact in any order and C must equal the INT8 oracle."""
    r = np.random.default_rng(5)
    M, N, K = 130, 200, 2048
    A = r.integers(-4, 5, (M, K))
    B = r.integers(-4, 5, (N, K))
    got = _run("f16", A.astype(np.float16), B.astype(np.float16), K)
    ref = oracle.gemm_i8(A.astype(np.int8), B.astype(np.int8))
    assert np.array_equal(got, ref.astype(np.float32))


def test_strided_operands_and_output():
    import torch
    M, N, K = 70, 90, 100
    for prec in ["i8", "f16", "i4"]:
        A, B = inputs.gemm_problem(prec, M, N, K, seed=9)
        pad = 64 if prec != "i4" else 32
        Ab = np.zeros((M, A.shape[1] + pad), dtype=A.dtype)
        Bb = np.zeros((N, B.shape[1] + pad), dtype=B.dtype)
        Ab[:, :A.shape[1]] = A
        Bb[:, :B.shape[1]] = B
        # garbage in the padding must not leak into C
        Ab[:, A.shape[1]:] = np.array(0x77, dtype=np.uint8).view(A.dtype) if A.dtype != np.float16 else np.float16(np.nan)
        Bb[:, B.shape[1]:] = np.array(0x77, dtype=np.uint8).view(B.dtype) if B.dtype != np.float16 else np.float16(np.nan)
        a = dev(Ab)[:, :A.shape[1]]
        b = dev(Bb)[:, :B.shape[1]]
        cdt = torch.float32 if prec == "f16" else torch.int32
        cbig = torch.full((M, N + 12), -1, dtype=cdt, device="cuda")
        c = cbig[:, :N]
        if prec == "i8":
            mp.gemm_i8(a, b, out=c)
        elif prec == "i4":
            mp.gemm_i4(a, b, K, out=c)
        else:
            mp.gemm_f16(a, b, out=c)
        whole = host(cbig)
        _compare(prec, whole[:, :N], _ref(prec, A, B, K), K, f"{prec} strided")
        assert np.all(whole[:, N:] == -1), "wrote past N"


# Output layouts of the epilogue: (row stride, first column) of C inside a
# larger buffer, with padding on both sides that must stay untouched: strides
# that are multiples of 4 and 16-byte aligned rows, a first column at an odd
# element, an odd stride; N = 90 is not a multiple of the 32-column blocks.
OUTPUT_LAYOUTS = [(96, 0), (96, 1), (93, 0), (100, 4)]


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("ldc,c0", OUTPUT_LAYOUTS)
def test_output_layouts(prec, ldc, c0):
    import torch
    M, N, K = 70, 90, 256
    A, B = inputs.gemm_problem(prec, M, N, K, seed=ldc + c0)
    cdt = torch.float32 if prec == "f16" else torch.int32
    cbig = torch.full((M, ldc), -1, dtype=cdt, device="cuda")
    c = cbig[:, c0:c0 + N]
    a, b = dev(A), dev(B)
    if prec == "i8":
        mp.gemm_i8(a, b, out=c)
    elif prec == "i4":
        mp.gemm_i4(a, b, K, out=c)
    else:
        mp.gemm_f16(a, b, out=c)
    whole = host(cbig)
    _compare(prec, whole[:, c0:c0 + N], _ref(prec, A, B, K), K, f"{prec} ldc {ldc} col {c0}")
    assert np.all(whole[:, :c0] == -1) and np.all(whole[:, c0 + N:] == -1), "wrote outside C"


@pytest.mark.parametrize("ldc,c0", OUTPUT_LAYOUTS)
def test_w4a4_output_layouts(ldc, c0):
    import torch
    M, N, K = 70, 90, 256
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=ldc + c0)
    ybig = torch.full((M, ldc), -1.0, dtype=torch.float16, device="cuda")
    mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b), out=ybig[:, c0:c0 + N])
    whole = host(ybig)
    _w4a4_check(A, B, K, sx, sw, b, whole[:, c0:c0 + N], f"w4a4 ldc {ldc} col {c0}")
    assert np.all(whole[:, :c0] == -1) and np.all(whole[:, c0 + N:] == -1), "wrote outside Y"


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
def test_unaligned_operands_byte_gather_path(prec):
    """Operands whose rows are not 16-byte aligned (odd strides, offset base)
    go through the byte-gather kernel."""
    M, N, K = 45, 77, 90
    A, B = inputs.gemm_problem(prec, M, N, K, seed=123)
    # shift the base by one element and use contiguous (unaligned) strides
    a_big = np.zeros((A.size + 8,), dtype=A.dtype)
    a_big[1:1 + A.size] = A.ravel()
    a = dev(a_big)[1:1 + A.size].view(A.shape[0], A.shape[1])
    b = dev(B)
    if prec == "i8":
        got = host(mp.gemm_i8(a, b))
    elif prec == "i4":
        got = host(mp.gemm_i4(a, b, K))
    else:
        got = host(mp.gemm_f16(a, b))
    _compare(prec, got, _ref(prec, A, B, K), K, f"{prec} unaligned")


def test_k_zero_writes_zeros():
    import torch
    h = mp.default_handle()
    a = torch.zeros((8, 16), dtype=torch.int8, device="cuda")
    c = torch.full((8, 8), 5, dtype=torch.int32, device="cuda")
    st = mp.mpgemm_run_i8(h, 8, 8, 0, a.data_ptr(), 16, a.data_ptr(), 16, c.data_ptr(), 8,
                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert np.all(host(c) == 0)


# ------------------------------------------------------------------ workload sizes

def _full_size(prec, cfg_index, n):
    """Every element of the GPU result against the oracle at the workload
    size. INT4 is compared with the INT8 oracle on the unpacked values (the
    INT4 oracle equals it exactly, a pinned invariant, and is ~30x slower);
    above N = 2048 an exact Freivalds check of the integer products is added
    as an independent second check."""
    A, B = inputs.gemm_problem(prec, n, n, n, inputs.config_seed(cfg_index, n))
    got = _run(prec, A, B, n)
    if prec == "i4":
        ref = oracle.gemm_i8(unpack_i4(A, n), unpack_i4(B, n))
    else:
        ref = _ref(prec, A, B, n)
    _compare(prec, got, ref, n, f"{prec} N={n} every element")
    del ref
    if n > 2048 and prec == "i8":
        freivalds_int(got, A, B, seed=n)
    elif n > 2048 and prec == "i4":
        freivalds_int(got, unpack_i4(A, n), unpack_i4(B, n), seed=n)


def test_int8_512_config0():
    _full_size("i8", 0, 512)


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096, 8192])
def test_fp16_square_config1(n):
    _full_size("f16", 1, n)


@pytest.mark.parametrize("n", [1024, 2048, 4096, 8192])
def test_int8_square_config2(n):
    _full_size("i8", 2, n)


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096, 8192])
def test_int4_square_config3(n):
    _full_size("i4", 3, n)


# ------------------------------------------------------------------ W4A16

def _w4(X, W, S, G):
    return host(mp.gemm_w4a16(dev(X), dev(W), dev(S), G)).view(np.uint16)


def _check_w4(X, W, S, K, G, what):
    got = _w4(X, W, S, G).view(np.float16).astype(np.float64)
    y, t2 = oracle.gemm_w4a16(X, W, S, K, G, want_t2=True)
    err = np.abs(got - y)
    tol = w4a16_tol(y, t2, K)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} outside the bar, worst {err.max()}"


@pytest.mark.parametrize("M", [1, 4, 16, 128])
def test_w4a16_config4(M):
    N = K = 4096
    G = 128
    X, W, S = inputs.w4a16_problem(M, N, K, G, inputs.config_seed(4, M))
    _check_w4(X, W, S, K, G, f"w4a16 M={M}")


@pytest.mark.parametrize("M,N,K,G", [(1, 16, 128, 128), (3, 50, 256, 128), (17, 70, 512, 128),
                                     (5, 33, 96, 32), (40, 130, 192, 64), (200, 64, 1024, 256),
                                     (2, 300, 4096, 4096)])
def test_w4a16_ragged(M, N, K, G):
    X, W, S = inputs.w4a16_problem(M, N, K, G, seed=M * 1000 + N + K + G)
    _check_w4(X, W, S, K, G, f"w4a16 {M}x{N}x{K} G={G}")


W4A16_CFGS = 21


@pytest.mark.parametrize("M,N,K,G", [(96, 4096, 4096, 128), (256, 4096, 4096, 128), (512, 4096, 4096, 128),
                                     (300, 200, 1440, 32), (640, 2048, 8192, 256)])
def test_w4a16_prefill_sizes(M, N, K, G):
    """M above 64 (but 128) runs the 128 x 64 ring kernel by default: K split
    over 4 workgroups (M = 96, a partial row block) or 2 (M = 256), no split
    (M = 512), ragged M with G = 32 and a partial last stage (K = 1440), 32
    stages per workgroup (K = 8192 in 2 slices); every element against the
    oracle."""
    X, W, S = inputs.w4a16_problem(M, N, K, G, seed=M + K + G)
    _check_w4(X, W, S, K, G, f"w4a16 {M}x{N}x{K} G={G}")


def test_w4a16_every_config(monkeypatch):
    """Each weight-only kernel configuration (forced through the ablation
    override) on ragged shapes, group sizes 32 ... 256 and the decode layer,
    plus the bit-exact small-integer cases (G = 64 and 128)."""
    shapes = [(1, 4096, 4096, 128), (1, 50, 96, 32), (2, 70, 512, 64), (3, 33, 256, 128),
              (5, 130, 1024, 256), (17, 40, 4096, 4096), (16, 4096, 4096, 128), (128, 1000, 4096, 128),
              (40, 200, 1440, 32), (130, 70, 640, 128), (2, 100, 6144, 128), (3, 64, 8192, 256)]
    problems = [(shape, inputs.w4a16_problem(*shape, seed=sum(shape) + 7)) for shape in shapes]
    refs = [oracle.gemm_w4a16(X, W, S, shape[2], shape[3], want_t2=True) for shape, (X, W, S) in problems]
    r = np.random.default_rng(5)
    Xi = r.integers(-4, 5, (3, 2048)).astype(np.float16)
    Wi = r.integers(0, 256, (96, 1024)).astype(np.uint8)
    Si = (2.0 ** -r.integers(3, 9, (96, 2048 // 64))).astype(np.float16)
    yi = oracle.f16_encode_rne_array(oracle.gemm_w4a16(Xi, Wi, Si, 2048, 64))
    # the same with G = 128 (the group size the matrix-unit GEMV needs)
    Si2 = (2.0 ** -r.integers(3, 9, (96, 2048 // 128))).astype(np.float16)
    yi2 = oracle.f16_encode_rne_array(oracle.gemm_w4a16(Xi, Wi, Si2, 2048, 128))
    for cfg in range(W4A16_CFGS):
        monkeypatch.setenv("MPGEMM_W4A16_CFG", str(cfg))
        with mp.Handle() as h:
            for ((M, N, K, G), (X, W, S)), (y, t2) in zip(problems, refs):
                xd, wd, sd = dev(X), dev(W), dev(S)
                got = host(mp.gemm_w4a16(xd, wd, sd, G, handle=h.value))
                err = np.abs(got.astype(np.float64) - y)
                bad = np.argwhere(err > w4a16_tol(y, t2, K))
                assert bad.size == 0, f"cfg {cfg} {M}x{N}x{K} G={G}: {len(bad)} outside the bar"
                # reproducible: the same call gives the same bits (split-K adds slices in a fixed order)
                again = host(mp.gemm_w4a16(xd, wd, sd, G, handle=h.value))
                assert np.array_equal(got.view(np.uint16), again.view(np.uint16)), f"cfg {cfg} {M}x{N}x{K}: not reproducible"
            got = host(mp.gemm_w4a16(dev(Xi), dev(Wi), dev(Si), 64, handle=h.value)).view(np.uint16)
            assert np.array_equal(got, yi), f"cfg {cfg}: small-integer case not bit-exact"
            # twice in a row: the split-K arrival counters must be back at zero
            got = host(mp.gemm_w4a16(dev(Xi), dev(Wi), dev(Si), 64, handle=h.value)).view(np.uint16)
            assert np.array_equal(got, yi), f"cfg {cfg}: second call differs"
            got = host(mp.gemm_w4a16(dev(Xi), dev(Wi), dev(Si2), 128, handle=h.value)).view(np.uint16)
            assert np.array_equal(got, yi2), f"cfg {cfg}: small-integer case (G = 128) not bit-exact"
            z = mp.gemm_w4a16(dev(np.zeros((3, 0), np.float16)), dev(np.zeros((5, 0), np.uint8)),
                              dev(np.zeros((5, 0), np.float16)), 32, handle=h.value)
            assert np.array_equal(host(z).astype(np.float64), np.zeros((3, 5))), f"cfg {cfg}: K = 0"


@pytest.mark.parametrize("G", [32, 128])
def test_w4a16_one_hot_exact(G):
    """x = e_k: y[n] = rne16(q[n,k] * s[n, k/G]) exactly (a single nonzero term)."""
    N, K = 48, 512
    _, W, S = inputs.w4a16_problem(1, N, K, G, seed=31)
    q = unpack_i4(W, K)
    ks = [0, 1, 7, 8, G - 1, G, G + 1, K - 1]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    got = _w4(X, W, S, G)
    for i, k in enumerate(ks):
        exact = q[:, k].astype(np.float64) * S[:, k // G].astype(np.float64)
        assert np.array_equal(got[i], oracle.f16_encode_rne_array(exact)), f"k={k}"


@pytest.mark.parametrize("M,G", [(1, 128), (2, 128), (4, 256), (16, 128), (128, 128), (16, 64)])
def test_w4a16_exact_small_integers(M, G):
    """Small-integer x and power-of-two scales: every partial sum is exact in
    fp32, so Y must be the fp16 rounding of the exact sum, bit for bit."""
    N, K = 256, 4096
    r = np.random.default_rng(M + G)
    X = r.integers(-4, 5, (M, K)).astype(np.float16)
    W = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    S = (2.0 ** -r.integers(3, 9, (N, K // G))).astype(np.float16)
    y = oracle.gemm_w4a16(X, W, S, K, G)
    assert np.array_equal(_w4(X, W, S, G), oracle.f16_encode_rne_array(y))


@pytest.mark.parametrize("M,N,K,G,cfg", [(9, 40, 256, 128, None), (200, 100, 1440, 32, 12), (150, 70, 512, 64, 12),
                                         (40, 72, 640, 128, 10), (3, 50, 1152, 128, None), (1, 50, 1152, 128, None)])
def test_w4a16_strided(M, N, K, G, cfg, monkeypatch):
    """Operands with padded rows (NaN activations and scales, 0x88 weights
    past K) and an output with padded columns: nothing past K or N is read
    into a result or written; for the default kernels at M = 9 (slice), 3
    (matrix-unit GEMV) and 1 (VALU GEMV), the ring kernel (ragged M, N and a
    partial last stage, K split over workgroups) and the slice kernel."""
    import torch
    if cfg is not None:
        monkeypatch.setenv("MPGEMM_W4A16_CFG", str(cfg))
    X, W, S = inputs.w4a16_problem(M, N, K, G, seed=3 + M)
    Xb = np.zeros((M, K + 64), np.float16); Xb[:, :K] = X; Xb[:, K:] = np.nan
    Wb = np.full((N, K // 2 + 32), 0x88, np.uint8); Wb[:, :K // 2] = W
    Sb = np.full((N, K // G + 5), np.nan, np.float16); Sb[:, :K // G] = S
    ybig = torch.full((M, N + 8), -7.0, dtype=torch.float16, device="cuda")
    with mp.Handle() as h:
        mp.gemm_w4a16(dev(Xb)[:, :K], dev(Wb)[:, :K // 2], dev(Sb)[:, :K // G], G, out=ybig[:, :N], handle=h.value)
    whole = host(ybig)
    y, t2 = oracle.gemm_w4a16(X, W, S, K, G, want_t2=True)
    assert np.all(np.abs(whole[:, :N].astype(np.float64) - y) <= w4a16_tol(y, t2, K))
    assert np.all(whole[:, N:] == -7.0)


# ------------------------------------------------------------------ W4A4: INT4 x INT4 with scale epilogue

def _w4a4_check(A, B, K, sx, sw, b, got, what):
    y = oracle.gemm_w4a4(A, B, K, sx, sw, b)
    # |integer product| for the bar: the INT8 oracle on the unpacked values
    # (equal to the INT4 oracle, and much faster)
    c_abs = np.abs(oracle.gemm_i8(unpack_i4(A, K), unpack_i4(B, K)).astype(np.float64))
    err = np.abs(got.astype(np.float64) - y)
    bad = np.argwhere(err > w4a4_tol(y, c_abs, sx, sw, b))
    assert bad.size == 0, f"{what}: {len(bad)} outside the bar, worst {err.max()}"


@pytest.mark.parametrize("M,N,K,with_bias", [(1, 1, 2, True), (64, 64, 128, True), (300, 520, 200, False),
                                             (257, 129, 4096, True), (1024, 1024, 1024, True)])
def test_w4a4_against_oracle(M, N, K, with_bias):
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=M + 3 * N + K)
    b = b if with_bias else None
    got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b) if b is not None else None))
    _w4a4_check(A, B, K, sx, sw, b, got, f"w4a4 {M}x{N}x{K}")


@pytest.mark.parametrize("K", [200, 512])
def test_w4a4_every_tile_config(K, monkeypatch):
    """Every tile configuration with the scale epilogue; K = 512 (256 bytes
    per row) also reaches the kernels that need whole 128-byte stages."""
    M, N = 300, 520
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=78 + K)
    for cfg in range(N_TILE_CFGS):
        monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        with mp.Handle() as h:
            got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b), handle=h.value))
        _w4a4_check(A, B, K, sx, sw, b, got, f"w4a4 cfg {cfg}")


def test_w4a4_exact_when_representable():
    """Power-of-two scales and integer bias: every output is exactly
    representable in fp16 (|y| < 2048), so Y must match bit for bit."""
    M, N, K = 96, 80, 64
    A, B, _, _, _ = inputs.w4a4_problem(M, N, K, seed=5)
    r = np.random.default_rng(6)
    sx = (2.0 ** -r.integers(0, 4, M)).astype(np.float16)
    sw = (2.0 ** -r.integers(0, 4, N)).astype(np.float16)
    b = r.integers(-16, 16, N).astype(np.float16)
    got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b))).view(np.uint16)
    want = oracle.f16_encode_rne_array(oracle.gemm_w4a4(A, B, K, sx, sw, b))
    assert np.array_equal(got, want)


def test_w4a4_epilogue_rounding_bits():
    """Non-power-of-two scales and a non-integer bias: Y must equal, bit for
    bit, the stated epilogue rounding: the exact integer product (from the
    oracle), times SX[m] in fp32, times SW[n] in fp32, plus bias[n] in fp32,
    each operation rounded on its own (no fused multiply-add), then fp16
    round-to-nearest-even. A fused multiply-add would differ in the last bit
    on a fraction of the outputs."""
    M, N, K = 1000, 1100, 512
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=21)
    r = np.random.default_rng(22)
    sx = r.uniform(0.003, 0.05, M).astype(np.float16)
    sw = r.uniform(0.003, 0.05, N).astype(np.float16)
    b = r.uniform(-3.0, 3.0, N).astype(np.float16)
    got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b))).view(np.uint16)
    acc = oracle.gemm_i8(unpack_i4(A, K), unpack_i4(B, K)).astype(np.float32)
    y = (acc * sx.astype(np.float32)[:, None]).astype(np.float32)
    y = (y * sw.astype(np.float32)[None, :]).astype(np.float32)
    y = (y + b.astype(np.float32)[None, :]).astype(np.float32)
    want = y.astype(np.float16).view(np.uint16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ from separately rounded fp32 steps, first {bad[:4].tolist()}"


def test_w4a4_strided_unaligned_and_k0():
    """Row strides beyond K, operands at an odd byte offset (byte-gather
    kernel), and K = 0 (Y = bias)."""
    import torch
    M, N, K = 70, 90, 160
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=8)
    Ab = np.zeros((M, K // 2 + 9), np.uint8); Ab[:, 1:1 + K // 2] = A
    Bb = np.zeros((N, K // 2 + 9), np.uint8); Bb[:, 1:1 + K // 2] = B
    got = host(mp.gemm_w4a4(dev(Ab)[:, 1:1 + K // 2], dev(Bb)[:, 1:1 + K // 2], K, dev(sx), dev(sw), dev(b)))
    _w4a4_check(A, B, K, sx, sw, b, got, "w4a4 strided/unaligned")
    z = host(mp.gemm_w4a4(dev(np.zeros((M, 0), np.uint8)), dev(np.zeros((N, 0), np.uint8)), 0,
                          dev(sx), dev(sw), dev(b)))
    assert np.array_equal(z.view(np.uint16), np.tile(b.view(np.uint16), (M, 1)))


def test_w4a4_full_size():
    """N = 4096: every element against the oracle. N = 8192: two rows in each
    256-row band of output tiles (their position in the band varies from band
    to band, so every wavefront row block and accumulator register of the
    tile is reached), every column of those rows."""
    n = 4096
    A, B, sx, sw, b = inputs.w4a4_problem(n, n, n, seed=n)
    got = host(mp.gemm_w4a4(dev(A), dev(B), n, dev(sx), dev(sw), dev(b)))
    _w4a4_check(A, B, n, sx, sw, b, got, f"w4a4 {n} every element")
    n = 8192
    A, B, sx, sw, b = inputs.w4a4_problem(n, n, n, seed=n)
    got = host(mp.gemm_w4a4(dev(A), dev(B), n, dev(sx), dev(sw), dev(b)))
    rows = band_rows(n, 256, per_band=2)
    _w4a4_check(A[rows], B, n, sx[rows], sw, b, got[rows], f"w4a4 {n} rows of every 256-row band")


# ------------------------------------------------------------------ INT4 weight quantisation

def _quant(W, G, h=None):
    q, sc = mp.quantize_w4(dev(W), G, handle=h)
    return host(q), host(sc).view(np.uint16)


@pytest.mark.parametrize("N,K,G", [(4096, 4096, 128), (37, 96, 32), (5, 640, 64), (8, 1536, 256),
                                   (3, 2048, 512), (1, 512, 512), (130, 4096, 32)])
def test_quantize_bit_exact(N, K, G):
    """Packed codes and fp16 scales identical to the oracle, bit for bit
    (4096 x 4096, G = 128 is the weight-only GEMM's layer)."""
    W = inputs.f16_weights(N * 7 + K + G, 0, N, K)
    Q, S = _quant(W, G)
    Qr, Sr = oracle.quantize_w4(W, G)
    assert np.array_equal(Q, Qr)
    assert np.array_equal(S, Sr.view(np.uint16))


def test_quantize_edge_values():
    """Zero groups, one nonzero weight, exact ties, subnormal and maximal
    fp16 weights."""
    G, K = 32, 256
    W = np.zeros((6, K), dtype=np.float64)
    W[1, 5] = -0.25                                    # single nonzero: q = -7
    W[2, :8] = np.array([7, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]) * 2.0 ** -4   # ties
    W[3, 32:64] = 2.0 ** -24 * np.arange(32)           # subnormals
    W[4, 64:96] = np.linspace(-65504, 65504, 32)       # extremes
    W[5] = np.random.default_rng(2).standard_normal(K)
    W = W.astype(np.float16)
    Q, S = _quant(W, G)
    Qr, Sr = oracle.quantize_w4(W, G)
    assert np.array_equal(Q, Qr)
    assert np.array_equal(S, Sr.view(np.uint16))
    assert np.all(S[0] == 0) and np.all(Q[0] == 0)


def test_quantize_many_ties():
    """Groups whose maximum is exactly 7 s with every other weight (k + 1/2) s:
    each of those quotients is an exact tie, resolved to the even code; scales
    with few mantissa bits over many exponents, K = 800 (a partial 512-k
    segment)."""
    N, K, G = 64, 800, 32
    r = np.random.default_rng(11)
    ng = K // G
    mant = r.integers(8, 64, (N, ng))                     # at most 6 significant bits
    expo = r.integers(-14, 6, (N, ng)).astype(np.float64)
    s = mant * 2.0 ** (expo - 5)
    k = r.integers(-7, 7, (N, K)).astype(np.float64)
    W = (k + 0.5) * np.repeat(s, G, axis=1)
    W[:, ::G] = 7 * s                                     # the group maximum
    W = W.astype(np.float16)
    assert np.all(np.isfinite(W))
    Q, S = _quant(W, G)
    Qr, Sr = oracle.quantize_w4(W, G)
    assert np.array_equal(S, Sr.view(np.uint16))
    assert np.array_equal(Q, Qr)


def test_quantize_strided_and_feeds_w4a16():
    """Row strides beyond K on every operand, bytes outside untouched; the
    quantised weights drive the weight-only GEMM to the oracle's result."""
    import torch
    N, K, G, M = 24, 512, 128, 3
    W = inputs.f16_weights(99, 0, N, K)
    Wb = np.full((N, K + 64), np.nan, np.float16); Wb[:, :K] = W
    qbig = torch.full((N, K // 2 + 16), 0x5A, dtype=torch.uint8, device="cuda")
    sbig = torch.full((N, K // G + 3), -3.0, dtype=torch.float16, device="cuda")
    mp.quantize_w4(dev(Wb)[:, :K], G, out_q=qbig[:, :K // 2], out_s=sbig[:, :K // G])
    Qr, Sr = oracle.quantize_w4(W, G)
    qh, sh = host(qbig), host(sbig)
    assert np.array_equal(qh[:, :K // 2], Qr) and np.all(qh[:, K // 2:] == 0x5A)
    assert np.array_equal(sh[:, :K // G].view(np.uint16), Sr.view(np.uint16)) and np.all(sh[:, K // G:] == -3.0)
    X = inputs.f16_normal(7, 0, M, K)
    y = host(mp.gemm_w4a16(dev(X), qbig[:, :K // 2], sbig[:, :K // G], G)).astype(np.float64)
    yr, t2 = oracle.gemm_w4a16(X, Qr, Sr, K, G, want_t2=True)
    assert np.all(np.abs(y - yr) <= w4a16_tol(yr, t2, K))


# ------------------------------------------------------------------ argument errors with a device

def test_argument_errors_with_handle():
    import torch
    h = mp.default_handle()
    a = torch.zeros((64, 64), dtype=torch.int8, device="cuda")
    c = torch.zeros((64, 64), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    A, C = a.data_ptr(), c.data_ptr()
    assert mp.mpgemm_run_i8(h, 64, 64, 64, A, 64, A, 64, C + 2, 64, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_run_i8(h, 64, 64, 64, A, 63, A, 64, C, 64, s) == mp.MPGEMM_ERR_INVALID_ARG
    assert mp.mpgemm_run_i4(h, 64, 64, 63, A, 64, A, 64, C, 64, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_run_i8(h, 64, 64, 200000, A, 200000, A, 200000, C, 64, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_run_w4a16(h, 1, 64, 64, A, 64, A, 64, A, 1, 48, C, 64, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_run_i8(h, 0, 64, 64, 0, 64, 0, 64, 0, 64, s) == mp.MPGEMM_OK
    torch.cuda.synchronize()
    assert np.all(host(c) == 0), "an argument error touched the output"
