"""Parity of the W4A4 call with the low-rank branch (mpgemm_run_w4a4_lowrank)
with the CPU oracle: Y = fp16((Q(X) Q(W)^T) (.) scale + L(X) + b) with
L(X) = fp16(X LD^T) LU^T ("Warp-Specialized Kernel Implementation for W4A4
MatMul on Latest GPU Architectures", section 1).

The bar adds to the W4A4 bar what the low-rank branch can differ by: U is an
fp32 sum on the GPU and exact in the oracle, so its fp16 rounding may land one
fp16 step apart (plus the fp32 sum's own error), and L's fp32 sum over the
rank has its own rounding error; the epilogue's two extra fp32 additions add
one rounding each.
"""
import numpy as np
import pytest

import oracle
import precision_dense_gemm_tiled_amd as mp
from precision_dense_gemm_tiled_amd import inputs
from tests.gpu_util import N_TILE_CFGS, band_rows, dev, host, require_gpu, unpack_i4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu(oracle_lib):
    require_gpu()
    return True


def _run(A, B, K, sx, sw, b, X, LD, LU, handle=None):
    return host(mp.gemm_w4a4_lowrank(dev(A), dev(B), K, dev(sx), dev(sw), dev(X), dev(LD), dev(LU),
                                     bias=dev(b) if b is not None else None, handle=handle))


def lowrank_ref_and_bar(A, B, K, sx, sw, b, X, LD, LU):
    """The oracle's Y (double, unrounded) and the per-element bar."""
    main = oracle.gemm_w4a4(A, B, K, sx, sw, None)
    U, L = oracle.w4a4_lowrank(X, LD, LU)
    bb = b.astype(np.float64)[None, :] if b is not None else 0.0
    y = main + L + bb
    R = LD.shape[0]
    f64 = lambda v: v.astype(np.float64)
    # |U|'s fp32 sum error (K products, each exact) and its fp16 rounding
    u_abs = np.abs(f64(X)) @ np.abs(f64(LD)).T
    du = max(K, 1) * 2.0 ** -24 * u_abs + 2.0 ** -10 * np.abs(U) + 2.0 ** -24
    lu = np.abs(f64(LU))
    dl = du @ lu.T + R * 2.0 ** -24 * ((np.abs(U) * (1 + 2.0 ** -10)) @ lu.T)
    c_abs = np.abs(oracle.gemm_i8(unpack_i4(A, K), unpack_i4(B, K)).astype(np.float64))
    mag = c_abs * np.abs(f64(sx))[:, None] * np.abs(f64(sw))[None, :]
    absb = np.abs(bb) if b is not None else 0.0
    bar = 2.0 ** -11 * np.abs(y) + 4 * 2.0 ** -24 * (mag + np.abs(L) + dl + absb) + dl + 2.0 ** -24
    return y, bar


def _check(A, B, K, sx, sw, b, X, LD, LU, got, what):
    y, bar = lowrank_ref_and_bar(A, B, K, sx, sw, b, X, LD, LU)
    err = np.abs(got.astype(np.float64) - y)
    bad = np.argwhere(err > bar)
    assert bad.size == 0, f"{what}: {len(bad)} outside the bar, first {bad[:4].tolist()}"


@pytest.mark.parametrize("M,N,K,R,with_bias", [
    (1, 1, 2, 16, True), (64, 64, 128, 32, True), (300, 520, 200, 16, False), (33, 700, 130, 48, True),
    (5, 17, 64, 128, True), (257, 129, 4096, 64, True), (1024, 1024, 1024, 256, True), (700, 300, 512, 32, False),
    (40, 100, 256, 48, True), (3, 50, 4096, 80, False), (8192, 64, 1024, 32, True)])
def test_lowrank_against_oracle(M, N, K, R, with_bias):
    """Ragged shapes, ranks in partial 32-rank blocks, a tall skinny case."""
    A, B, sx, sw, b, X, LD, LU = inputs.w4a4_lowrank_problem(M, N, K, R, seed=M + 3 * N + K + R)
    b = b if with_bias else None
    got = _run(A, B, K, sx, sw, b, X, LD, LU)
    _check(A, B, K, sx, sw, b, X, LD, LU, got, f"w4a4 low-rank {M}x{N}x{K} R={R}")


def test_lowrank_random_shapes_reproducible():
    """Twelve seeded random shapes (M, N up to 700, K a multiple of 2 up to
    2048, R a multiple of 16 up to 128): against the oracle, and a second call
    with the same inputs gives the same bits."""
    r = np.random.default_rng(2026)
    for i in range(12):
        M, N = int(r.integers(1, 701)), int(r.integers(1, 701))
        K = 2 * int(r.integers(1, 1025)) if i % 3 else 64 * int(r.integers(1, 33))
        R = 16 * int(r.integers(1, 9))
        A, B, sx, sw, b, X, LD, LU = inputs.w4a4_lowrank_problem(M, N, K, R, seed=300 + i)
        got = _run(A, B, K, sx, sw, b, X, LD, LU)
        _check(A, B, K, sx, sw, b, X, LD, LU, got, f"w4a4 low-rank {M}x{N}x{K} R={R}")
        again = _run(A, B, K, sx, sw, b, X, LD, LU)
        assert np.array_equal(got.view(np.uint16), again.view(np.uint16)), f"{M}x{N}x{K} R={R}: not reproducible"


def test_lowrank_every_tile_config(monkeypatch):
    """Every tile configuration (forced for both launches: the FP16 down-
    projection and the W4A4 kernel with the low-rank epilogue); K = 512 also
    reaches the kernels that need whole 128-byte stages; twice per
    configuration, bit-identical."""
    M, N, K, R = 300, 520, 512, 32
    A, B, sx, sw, b, X, LD, LU = inputs.w4a4_lowrank_problem(M, N, K, R, seed=91)
    for cfg in range(N_TILE_CFGS):
        monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        with mp.Handle() as h:
            got = _run(A, B, K, sx, sw, b, X, LD, LU, handle=h.value)
            again = _run(A, B, K, sx, sw, b, X, LD, LU, handle=h.value)
        _check(A, B, K, sx, sw, b, X, LD, LU, got, f"w4a4 low-rank cfg {cfg}")
        assert np.array_equal(got.view(np.uint16), again.view(np.uint16)), f"cfg {cfg}: not reproducible"


def _exact_inputs(M, N, K, R, seed):
    """Inputs for which every fp32 step of the branch is exact: integer X in
    [-4, 4], LD in {-1/4, 0, 1/4} (U a multiple of 1/4, |U| <= K, exact in
    fp16), LU = +-2^-e (e in 0 ... 6), so every partial sum of L is a multiple
    of 2^-8 below 2^22 * 2^-8."""
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=seed)
    r = np.random.default_rng(seed)
    X = r.integers(-4, 5, (M, K)).astype(np.float16)
    LD = (r.integers(-1, 2, (R, K)) * 0.25).astype(np.float16)
    LU = (r.choice([-1.0, 1.0], (N, R)) * 2.0 ** -r.integers(0, 7, (N, R))).astype(np.float16)
    return A, B, sx, sw, b, X, LD, LU


def test_lowrank_exact_when_representable():
    """Power-of-two scales, integer bias and an exact branch: every output is
    an exact multiple of 2^-8 below 2^11, so Y must match bit for bit."""
    M, N, K, R = 96, 80, 64, 32
    A, B, _, _, _, X, LD, LU = _exact_inputs(M, N, K, R, seed=5)
    r = np.random.default_rng(6)
    sx = (2.0 ** -r.integers(0, 4, M)).astype(np.float16)
    sw = (2.0 ** -r.integers(0, 4, N)).astype(np.float16)
    b = r.integers(-16, 16, N).astype(np.float16)
    got = _run(A, B, K, sx, sw, b, X, LD, LU).view(np.uint16)
    _, L = oracle.w4a4_lowrank(X, LD, LU)
    y = oracle.gemm_w4a4(A, B, K, sx, sw, b) + L
    assert np.all(np.abs(y) < 2048) and np.all(y * 256 == np.round(y * 256))
    assert np.array_equal(got, oracle.f16_encode_rne_array(y))


def test_lowrank_epilogue_rounding_bits():
    """Non-power-of-two scales and bias with an exact branch: Y must equal,
    bit for bit, the stated order: ((acc * SX) * SW + L) + bias, each fp32
    operation rounded on its own, then fp16 round-to-nearest-even."""
    M, N, K, R = 600, 700, 512, 32
    A, B, _, _, _, X, LD, LU = _exact_inputs(M, N, K, R, seed=23)
    r = np.random.default_rng(24)
    sx = r.uniform(0.003, 0.05, M).astype(np.float16)
    sw = r.uniform(0.003, 0.05, N).astype(np.float16)
    b = r.uniform(-3.0, 3.0, N).astype(np.float16)
    got = _run(A, B, K, sx, sw, b, X, LD, LU).view(np.uint16)
    _, L = oracle.w4a4_lowrank(X, LD, LU)
    assert np.array_equal(L.astype(np.float32).astype(np.float64), L), "the branch must be exact in fp32"
    acc = oracle.gemm_i8(unpack_i4(A, K), unpack_i4(B, K)).astype(np.float32)
    y = (acc * sx.astype(np.float32)[:, None]).astype(np.float32)
    y = (y * sw.astype(np.float32)[None, :]).astype(np.float32)
    y = (y + L.astype(np.float32)).astype(np.float32)
    y = (y + b.astype(np.float32)[None, :]).astype(np.float32)
    want = y.astype(np.float16).view(np.uint16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ from the separately rounded fp32 steps, first {bad[:4].tolist()}"


def test_lowrank_rounds_u_to_fp16():
    """U[m][0] = 1 + 2^-10 + 2^-11 (a tie between two fp16 values, exact in
    fp32) becomes 1 + 2^-9 before the up-projection; U[m][1] = 1. With
    LU[n] = (1, -1, 0, ...) and a zero INT4 product, Y = fp16(U16[0] - U16[1])
    = 2^-9 exactly; an unrounded U would give 1.5 * 2^-10."""
    M, N, K, R = 3, 5, 64, 16
    A = np.zeros((M, K // 2), np.uint8)
    B = np.zeros((N, K // 2), np.uint8)
    X = np.zeros((M, K), np.float16)
    X[:, 0] = 1 + 2 ** -10
    X[:, 1] = 2 ** -11
    X[:, 2] = 1
    LD = np.zeros((R, K), np.float16)
    LD[0, 0] = LD[0, 1] = 1
    LD[1, 2] = 1
    LU = np.zeros((N, R), np.float16)
    LU[:, 0], LU[:, 1] = 1, -1
    ones_m, ones_n = np.ones(M, np.float16), np.ones(N, np.float16)
    got = _run(A, B, K, ones_m, ones_n, None, X, LD, LU).view(np.uint16)
    assert np.all(got == np.float16(2 ** -9).view(np.uint16))
    assert np.float16(1.5 * 2 ** -10) != np.float16(2 ** -9)


def test_lowrank_rank0_strided_and_k0():
    """R = 0 is the plain W4A4 call (identical bits); strided X, LD and LU
    views and an output inside a larger buffer (padding untouched); K = 0
    gives Y = fp16(L + bias) = bias (U = 0)."""
    import torch
    M, N, K, R = 70, 90, 160, 32
    A, B, sx, sw, b, X, LD, LU = inputs.w4a4_lowrank_problem(M, N, K, R, seed=17)
    plain = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b)))
    r0 = host(mp.gemm_w4a4_lowrank(dev(A), dev(B), K, dev(sx), dev(sw), dev(X), dev(LD[:0]), dev(LU[:, :0]),
                                   bias=dev(b)))
    assert np.array_equal(r0.view(np.uint16), plain.view(np.uint16))
    Xb = np.zeros((M, K + 24), np.float16); Xb[:, 3:3 + K] = X
    LDb = np.zeros((R, K + 8), np.float16); LDb[:, :K] = LD
    LUb = np.zeros((N, R + 8), np.float16); LUb[:, :R] = LU
    Yb = torch.full((M, N + 6), -7.0, dtype=torch.float16, device="cuda")
    mp.gemm_w4a4_lowrank(dev(A), dev(B), K, dev(sx), dev(sw), dev(Xb)[:, 3:3 + K], dev(LDb)[:, :K],
                         dev(LUb)[:, :R], bias=dev(b), out=Yb[:, 2:2 + N])
    yb = host(Yb)
    assert np.all(yb[:, :2] == -7.0) and np.all(yb[:, 2 + N:] == -7.0)
    _check(A, B, K, sx, sw, b, X, LD, LU, yb[:, 2:2 + N], "w4a4 low-rank strided")
    z = host(mp.gemm_w4a4_lowrank(dev(np.zeros((M, 0), np.uint8)), dev(np.zeros((N, 0), np.uint8)), 0, dev(sx),
                                  dev(sw), dev(np.zeros((M, 0), np.float16)), dev(np.zeros((R, 0), np.float16)),
                                  dev(LU), bias=dev(b)))
    assert np.array_equal(z.view(np.uint16), np.tile(b.view(np.uint16), (M, 1)))


def test_lowrank_full_size():
    """N = 4096, R = 32 (the benchmark's shape): two rows in each 256-row band
    of output tiles, every column of those rows, against the oracle."""
    n, R = 4096, 32
    A, B, sx, sw, b, X, LD, LU = inputs.w4a4_lowrank_problem(n, n, n, R, seed=n + R)
    got = _run(A, B, n, sx, sw, b, X, LD, LU)
    rows = band_rows(n, 256, per_band=2)
    _check(A[rows], B, n, sx[rows], sw, b, X[rows], LD, LU, got[rows], f"w4a4 low-rank {n} rows of every band")
