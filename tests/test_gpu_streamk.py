"""Stream-K tile scheduling on the GPU (through the C-ABI) against the oracle.

A stream-K launch splits the K loops of some tiles over several workgroups
and sums their partial tiles in a fixed order, so integer results must still
match the oracle bit for bit, FP16 within the stated bar, and repeated calls
(and graph replays) must be bit-identical. MPGEMM_STREAMK=1 forces the split
on every configuration whose tiles do not fill whole waves; without it the
library splits only a short last wave.
"""
import numpy as np
import pytest

import oracle
import precision_dense_gemm_tiled_amd as mp
from precision_dense_gemm_tiled_amd import inputs
from tests.gpu_util import N_TILE_CFGS, dev, f16_tol, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu(oracle_lib):
    require_gpu()
    return True


def _run(prec, A, B, K, h):
    a, b = dev(A), dev(B)
    if prec == "i8":
        return host(mp.gemm_i8(a, b, handle=h))
    if prec == "i4":
        return host(mp.gemm_i4(a, b, K, handle=h))
    return host(mp.gemm_f16(a, b, handle=h))


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


# K = 992: a partial K tile for every precision and stage depth (f16: 15.5
# stages of 128 bytes, i8: 7.75, i4: 3.875), 16-byte aligned rows throughout.
@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
def test_every_tile_config_forced(prec, monkeypatch):
    """300 x 520 outputs: 6 to 90 tiles, far below one wave, so every K
    iteration of every tile gets a workgroup of its own or shares one with a
    neighbour: up to 16 contributors per tile, ragged edges, the K tail in
    the first contributor's segment."""
    M, N, K = 300, 520, 992
    A, B = inputs.gemm_problem(prec, M, N, K, seed=91)
    ref = _ref(prec, A, B, K)
    monkeypatch.setenv("MPGEMM_STREAMK", "1")
    for cfg in range(N_TILE_CFGS):
        monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        with mp.Handle() as h:
            got = _run(prec, A, B, K, h.value)
            # the arrival counters are back at zero: a second call on the
            # same handle is just as correct, and bit-identical
            again = _run(prec, A, B, K, h.value)
        _compare(prec, got, ref, K, f"{prec} cfg {cfg} stream-K")
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), f"{prec} cfg {cfg} repeat"


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (37, 70, 4096), (513, 260, 96), (129, 1025, 1312)])
def test_forced_shapes(prec, M, N, K, monkeypatch):
    """Degenerate and ragged shapes with the default tile choice: one output,
    few tiles with a long K, short K (2-3 stages), odd tile counts."""
    A, B = inputs.gemm_problem(prec, M, N, K, seed=M + 5 * N + 11 * K)
    monkeypatch.setenv("MPGEMM_STREAMK", "1")
    with mp.Handle() as h:
        got = _run(prec, A, B, K, h.value)
    _compare(prec, got, _ref(prec, A, B, K), K, f"{prec} {M}x{N}x{K} stream-K")


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
def test_auto_plan_splits_a_long_k(prec, monkeypatch):
    """256 x 256 x 32768: 16 tiles of 64 x 64, 128 to 512 K stages each; the
    default plan splits every tile over the grid. Every element is compared
    with the oracle, and with the data-parallel launch (integers bit for bit)."""
    M = N = 256
    K = 32768
    st, cfg, grid, tdp = mp.mpgemm_plan_gemm({"f16": 0, "i8": 1, "i4": 2}[prec], M, N, K, 256)
    assert st == 0 and grid > 0 and tdp == 0, (cfg, grid, tdp)
    A, B = inputs.gemm_problem(prec, M, N, K, seed=256)
    with mp.Handle() as h:
        got = _run(prec, A, B, K, h.value)
    monkeypatch.setenv("MPGEMM_STREAMK", "0")
    with mp.Handle() as h:
        dp = _run(prec, A, B, K, h.value)
    _compare(prec, got, _ref(prec, A, B, K), K, f"{prec} {M}x{N}x{K} split")
    if prec == "f16":
        err = np.abs(got.astype(np.float64) - dp.astype(np.float64))
        assert np.all(err <= 2 * f16_tol(K))
    else:
        assert np.array_equal(got, dp)


@pytest.mark.parametrize("prec", ["i8", "i4", "f16"])
@pytest.mark.parametrize("M,N,K", [(1100, 1300, 992), (300, 520, 4096), (2048, 2048, 2048)])
def test_persistent_whole_tiles(prec, M, N, K, monkeypatch):
    """MPGEMM_STREAMK=2: the stream-K kernel with every tile whole on a
    persistent grid of the resident workgroups (each loops over several
    tiles at 1100 x 1300 with 64 x 64 tiles and at 2048^2; fewer tiles than
    workgroups at 300 x 520), on every tile configuration at 2048^2 and with
    the default choice otherwise: the oracle's result, and for the integer
    precisions the one-tile-per-workgroup launch's bit for bit. (FP16 may
    differ from it in the last bits where a configuration's own kernel is not
    the ring kernel: the persistent grid always runs the ring kernel.)"""
    A, B = inputs.gemm_problem(prec, M, N, K, seed=M + N + K)
    ref = _ref(prec, A, B, K)
    cfgs = range(N_TILE_CFGS) if M == 2048 else [None]
    for cfg in cfgs:
        if cfg is not None:
            monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        monkeypatch.setenv("MPGEMM_STREAMK", "2")
        with mp.Handle() as h:
            got = _run(prec, A, B, K, h.value)
        _compare(prec, got, ref, K, f"{prec} {M}x{N}x{K} cfg {cfg} persistent")
        if prec != "f16":
            monkeypatch.setenv("MPGEMM_STREAMK", "0")
            with mp.Handle() as h:
                dp = _run(prec, A, B, K, h.value)
            assert np.array_equal(got, dp), f"{prec} cfg {cfg} persistent vs per-tile"


def test_graph_replays_match_eager(monkeypatch):
    """A stream-K launch captured in a HIP graph: every replay (with eager work
    and synchronisation in between) gives the eager result bit for bit."""
    import torch
    M, N, K = 600, 700, 2048
    A, B = inputs.gemm_problem("f16", M, N, K, seed=3)
    monkeypatch.setenv("MPGEMM_STREAMK", "1")
    with mp.Handle() as h:
        a, b = dev(A), dev(B)
        eager = host(mp.gemm_f16(a, b, handle=h.value))
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            mp.gemm_f16(a, b, out=out, handle=h.value)   # warm-up outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            mp.gemm_f16(a, b, out=out, handle=h.value)
        for i in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(out), eager), f"replay {i}"
            mp.gemm_f16(a, b, handle=h.value)   # eager work between replays
            torch.cuda.synchronize()
    _compare("f16", eager, oracle.gemm_f16(A, B), K, "graph eager")


def test_w4a4_every_tile_config_forced(monkeypatch):
    """The scale epilogue runs in the workgroup that finishes a split tile."""
    M, N, K = 300, 520, 992
    A, B, sx, sw, b = inputs.w4a4_problem(M, N, K, seed=79)
    y = oracle.gemm_w4a4(A, B, K, sx, sw, b)
    c_abs = np.abs(oracle.gemm_i4(A, B, K).astype(np.float64))
    mag = c_abs * np.abs(sx.astype(np.float64))[:, None] * np.abs(sw.astype(np.float64))[None, :]
    tol = 2.0 ** -11 * np.abs(y) + 3 * 2.0 ** -24 * (mag + np.abs(b.astype(np.float64))[None, :]) + 2.0 ** -24
    monkeypatch.setenv("MPGEMM_STREAMK", "1")
    for cfg in range(N_TILE_CFGS):
        monkeypatch.setenv("MPGEMM_TILE_CFG", str(cfg))
        with mp.Handle() as h:
            got = host(mp.gemm_w4a4(dev(A), dev(B), K, dev(sx), dev(sw), dev(b), handle=h.value))
        err = np.abs(got.astype(np.float64) - y)
        assert np.all(err <= tol), f"w4a4 cfg {cfg} stream-K: worst {err.max()}"
