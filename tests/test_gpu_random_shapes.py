"""Seeded random shapes through every default path, against the CPU oracle.

The hand-picked shapes of the other parity tests follow the kernels' tile
sizes; these draw (M, N, K, group size) from a fixed generator instead, so
that the planner's choices (the decode GEMVs, the slice and ring kernels, the
K splits, stream-K) meet shapes nobody chose for them. Every element is
compared with the oracle, to the same bars as the other parity tests.
"""
import numpy as np
import pytest

import oracle
import precision_dense_gemm_tiled_amd as mp
from precision_dense_gemm_tiled_amd import inputs
from tests.gpu_util import dev, f16_tol, host, require_gpu, unpack_i4, w4a4_tol, w4a16_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu(oracle_lib):
    require_gpu()
    return True


def _w4a16_shapes(count, seed):
    """M mostly in the decode range (1 ... 4), else up to 320; N up to 700;
    G a power of two in [32, 512]; K a multiple of G up to 4096."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        band = r.integers(0, 10)
        M = int(r.integers(1, 5) if band < 4 else r.integers(5, 65) if band < 7 else r.integers(65, 321))
        N = int(r.integers(1, 701))
        G = int(2 ** r.integers(5, 10))
        K = G * int(r.integers(1, 4096 // G + 1))
        out.append((M, N, K, G))
    return out


W4A16_SHAPES = _w4a16_shapes(36, 20261202)


@pytest.mark.parametrize("M,N,K,G", W4A16_SHAPES)
def test_w4a16_random_shape(M, N, K, G):
    """The default plan, and the allocation-free entry point (the same plan:
    identical bits)."""
    X, W, S = inputs.w4a16_problem(M, N, K, G, seed=M * 7919 + N * 31 + K + G)
    xd, wd, sd = dev(X), dev(W), dev(S)
    got = host(mp.gemm_w4a16(xd, wd, sd, G))
    y, t2 = oracle.gemm_w4a16(X, W, S, K, G, want_t2=True)
    err = np.abs(got.astype(np.float64) - y)
    bad = np.argwhere(err > w4a16_tol(y, t2, K))
    assert bad.size == 0, f"w4a16 {M}x{N}x{K} G={G}: {len(bad)} outside the bar, first {bad[:4].tolist()}"
    na = host(mp.gemm_w4a16_noalloc(xd, wd, sd, G))
    assert np.array_equal(na.view(np.uint16), got.view(np.uint16)), "allocation-free call differs"


def _gemm_shapes(count, seed, even_k):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(r.integers(1, 1101))
        N = int(r.integers(1, 1101))
        K = int(r.integers(1, 1537))
        if even_k:
            K += K & 1
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
def test_gemm_random_shapes(prec):
    """Twelve random (M, N, K) per precision, M and N up to 1100 (partial
    tiles on both edges, grids from one tile to a few hundred), K up to 1536
    (even for INT4)."""
    for i, (M, N, K) in enumerate(_gemm_shapes(12, {"f16": 11, "i8": 12, "i4": 13}[prec], prec == "i4")):
        A, B = inputs.gemm_problem(prec, M, N, K, seed=1000 * i + M + N + K)
        if prec == "i8":
            got, ref = host(mp.gemm_i8(dev(A), dev(B))), oracle.gemm_i8(A, B)
        elif prec == "i4":
            got, ref = host(mp.gemm_i4(dev(A), dev(B), K)), oracle.gemm_i4(A, B, K)
        else:
            got, ref = host(mp.gemm_f16(dev(A), dev(B))), oracle.gemm_f16(A, B)
        if prec == "f16":
            err = np.abs(got.astype(np.float64) - ref)
            assert np.all(err <= f16_tol(K)), f"f16 {M}x{N}x{K}: max err {err.max()}"
        else:
            bad = np.argwhere(got != ref)
            assert bad.size == 0, f"{prec} {M}x{N}x{K}: {len(bad)} mismatches, first {bad[:4].tolist()}"


def test_w4a4_random_shapes():
    """Ten random W4A4 shapes (even K), with and without the bias, to the W4A4
    bar of the other parity tests."""
    r = np.random.default_rng(14)
    for i in range(10):
        M, N = int(r.integers(1, 700)), int(r.integers(1, 700))
        K = 2 * int(r.integers(1, 769))
        A, B, sx, sw, bias = inputs.w4a4_problem(M, N, K, seed=77 * i + K)
        b = bias if i % 2 else None
        got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b) if b is not None else None))
        y = oracle.gemm_w4a4(A, B, K, sx, sw, b)
        c_abs = np.abs(oracle.gemm_i8(unpack_i4(A, K), unpack_i4(B, K)).astype(np.float64))
        err = np.abs(got.astype(np.float64) - y)
        bad = np.argwhere(err > w4a4_tol(y, c_abs, sx, sw, b))
        assert bad.size == 0, f"w4a4 {M}x{N}x{K}: {len(bad)} outside the bar, first {bad[:4].tolist()}"


def test_quantize_random_shapes():
    """Twenty random quantiser shapes (N up to 300, G in [32, 512], K a
    multiple of G up to 4096) and weight spreads from 1e-4 to 10: codes and
    scales identical to the oracle, bit for bit."""
    r = np.random.default_rng(15)
    for i in range(20):
        N = int(r.integers(1, 301))
        G = int(2 ** r.integers(5, 10))
        K = G * int(r.integers(1, 4096 // G + 1))
        std = float(10.0 ** r.uniform(-4, 1))
        W = inputs.f16_weights(500 + i, 0, N, K, std=std)
        q, s = mp.quantize_w4(dev(W), G)
        Qr, Sr = oracle.quantize_w4(W, G)
        assert np.array_equal(host(q), Qr), f"quantize {N}x{K} G={G} std={std:.3g}: codes differ"
        assert np.array_equal(host(s).view(np.uint16), Sr.view(np.uint16)), f"quantize {N}x{K} G={G}: scales differ"
