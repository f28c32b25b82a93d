"""Host-side planning of the library (no device): which tile configuration a
GEMM runs and how a weight-only call splits K. These decide grid shapes and
workspace use, so their invariants are checked here on many sizes."""
import os

import numpy as np
import pytest

OK, INVALID = 0, 1
# slice configurations of the weight-only path: (BM, BN, K held by one workgroup)
SLICE = {8: (16, 16, 4096), 9: (32, 32, 2048), 10: (64, 128, 1024), 11: (128, 128, 512),
         12: (128, 64, 128 * 95), 13: (128, 64, 128 * 31), 14: (64, 128, 512)}
WORKSPACE_FLOATS = 8 << 20


@pytest.fixture(scope="module")
def mp():
    import precision_dense_gemm_tiled_amd as mp
    if not os.path.exists(mp.lib_path):
        from precision_dense_gemm_tiled_amd import build
        build.build()
    mp.lib()
    return mp


@pytest.mark.parametrize("prec", [0, 1, 2, 3])
def test_tile_config_at_the_workload_sizes(mp, prec):
    """Square sizes of the benchmark on 256 compute units: 64x64 tiles at 512
    and 1024 (FP16 at 1024, 16 K stages: the 8-stage ring), 128x128 with a
    4-stage ring at 2048, 256x256 from 4096 on."""
    want = {512: 2, 1024: 22 if prec == 0 else 2, 2048: 6, 4096: 4, 8192: 4}
    for n, cfg in want.items():
        # whole waves of tiles (or a grid below one wave): data-parallel
        assert mp.mpgemm_plan_gemm(prec, n, n, n, 256) == (OK, cfg, 0, 0), n


def test_tile_config_fills_the_compute_units(mp):
    """Whatever is chosen, the grid has at least half as many tiles as compute
    units, or the smallest tile is chosen."""
    tiles = {0: 256, 1: 128, 2: 64, 3: 256, 4: 256, 5: 128, 6: 128}   # BM (= BN for the square ones)
    rng = np.random.default_rng(0)
    for _ in range(500):
        M, N, K = (int(v) for v in rng.integers(1, 20000, 3))
        st, cfg, _, _ = mp.mpgemm_plan_gemm(1, M, N, K, 256)
        assert st == OK and cfg in (2, 3, 4, 6)
        if cfg != 2:
            bm = tiles[cfg]
            bn = 128 if cfg == 3 else bm
            assert -(-M // bm) * -(-N // bn) >= 128


# tile configurations: (BM, BN, K bytes per stage, workgroups per compute unit)
TILE = {0: (256, 256, 64, 1), 1: (128, 128, 64, 2), 2: (64, 64, 128, 3), 3: (256, 128, 128, 1),
        4: (256, 256, 128, 1), 5: (128, 256, 128, 1), 6: (128, 128, 128, 1), 22: (64, 64, 128, 1)}
KBYTES = {0: lambda K: 2 * K, 1: lambda K: K, 2: lambda K: K // 2, 3: lambda K: K // 2}
WORKSPACE_BYTES = 128 << 20


def sk_partition(tiles_sk, KT, grid):
    """Segments (workgroup, tile, first entry, end entry, slot) of the stream-K
    part, with the ranges and slot rule of the kernel: workgroup w runs
    iterations [w I / G, (w+1) I / G); a partial tile goes to slot 0 when the
    workgroup's range starts inside it, else slot 1."""
    I = tiles_sk * KT
    segs = []
    for w in range(grid):
        beg, end = I * w // grid, I * (w + 1) // grid
        it = beg
        while it < end:
            t, e0 = divmod(it, KT)
            e1 = min(KT, e0 + end - it)
            slot = 0 if beg >= t * KT else 1
            segs.append((w, t, e0, e1, slot))
            it += e1 - e0
    return segs


def owner(x, I, grid):
    return ((x + 1) * grid - 1) // I


def test_stream_k_partition_invariants():
    """Every K iteration of every split tile is run exactly once, a workgroup
    has at most two partial tiles and they use distinct workspace slots, and
    the contributors of a tile are the contiguous workgroups the kernel's
    owner formula names."""
    rng = np.random.default_rng(2)
    cases = [(1, 2, 1), (3, 7, 5), (16, 10, 160), (289, 64, 256), (300, 33, 256)]
    cases += [(int(rng.integers(1, 600)), int(rng.integers(2, 80)), 0) for _ in range(300)]
    for tiles_sk, KT, grid in cases:
        I = tiles_sk * KT
        if grid == 0:
            grid = int(rng.integers(1, 600))
        grid = min(grid, I)
        segs = sk_partition(tiles_sk, KT, grid)
        cover = np.zeros(I, np.int64)
        used = set()
        for w, t, e0, e1, slot in segs:
            assert 0 <= e0 < e1 <= KT
            cover[t * KT + e0:t * KT + e1] += 1
            if not (e0 == 0 and e1 == KT):
                assert (w, slot) not in used
                used.add((w, slot))
        assert (cover == 1).all()
        by_tile = {}
        for w, t, e0, e1, slot in segs:
            by_tile.setdefault(t, []).append(w)
        for t, ws in by_tile.items():
            lo, hi = owner(t * KT, I, grid), owner(t * KT + KT - 1, I, grid)
            assert ws == list(range(lo, hi + 1)), (tiles_sk, KT, grid, t)


def test_stream_k_plan(mp):
    """Auto policy: a stream-K grid only when the tiles fill at most an eighth
    of the resident workgroups and each tile has at least 128 K stages; then
    every tile is split (no data-parallel part) over min(iterations, G)
    workgroups, and the partial tiles fit the handle's workspace."""
    rng = np.random.default_rng(3)
    seen = 0
    for i in range(3000):
        prec = int(rng.integers(0, 4))
        if i % 2:   # small outputs with long K, where splitting can pay
            M, N = (int(v) for v in rng.integers(1, 1500, 2))
            K = int(rng.integers(1, 40000)) * 2
        else:
            M, N = (int(v) for v in rng.integers(1, 12000, 2))
            K = int(rng.integers(1, 9000)) * 2
        st, cfg, grid, tdp = mp.mpgemm_plan_gemm(prec, M, N, K, 256)
        assert st == OK
        BM, BN, BKB, per_cu = TILE[cfg]
        T = -(-M // BM) * -(-N // BN)
        G = 256 * per_cu
        KT = -(-KBYTES[prec](K) // BKB)
        if grid == 0:
            assert tdp == 0
            assert 8 * T > G or KT < 128 or KBYTES[prec](K) < BKB
            continue
        seen += 1
        assert 8 * T <= G and KT >= 128
        assert tdp == 0 and grid == min(T * KT, G)
        assert 2 * grid * BM * BN * 4 <= WORKSPACE_BYTES
    assert seen > 20


def test_stream_k_policy_examples(mp):
    """N = 6144 FP16 (2.25 waves of 256 x 256 tiles) and N = 4352 INT8 (1.13
    waves) run data-parallel: splitting the short last wave was measured
    slower. 256 x 256 x 65536 INT8 (16 tiles of 64 x 64, 512 stages each) is
    split over all 768 resident workgroups."""
    assert mp.mpgemm_plan_gemm(0, 6144, 6144, 6144, 256) == (OK, 4, 0, 0)
    assert mp.mpgemm_plan_gemm(1, 4352, 4352, 4352, 256) == (OK, 4, 0, 0)
    assert mp.mpgemm_plan_gemm(1, 256, 256, 65536, 256) == (OK, 2, 768, 0)


def test_plan_gemm_arguments(mp):
    assert mp.mpgemm_plan_gemm(4, 8, 8, 8, 256)[0] == INVALID
    assert mp.mpgemm_plan_gemm(0, -1, 8, 8, 256)[0] == INVALID
    assert mp.mpgemm_plan_gemm(0, 8, 8, 8, 0)[0] == INVALID


def test_w4a16_plan_at_the_workload_sizes(mp):
    """N = K = 4096: the VALU GEMV for M = 1 (2 rows per wavefront), the
    matrix-unit GEMV for M = 2 ... 4 (16 rows per workgroup), 16 x 16 slices with K inside the workgroup at M = 16, 32 x 32 slices with K
    split in 2 at M = 32, 64 x 128 slices over 4 stages with K split in 8 at
    M = 33 ... 64, 64 x 128 slices with K split in 4 at M = 65 ... 128;
    above 128 rows, the 128 x 64 ring kernel, K split until the grid covers
    the 256 compute units (M = 256: 128 tiles, 2 slices; M >= 512: no
    split)."""
    want = {1: (3, 1), 2: (16, 1), 4: (16, 1), 16: (8, 1), 32: (9, 2), 33: (14, 8), 64: (14, 8), 65: (10, 4),
            96: (10, 4),
            127: (10, 4), 128: (10, 4), 129: (12, 2), 192: (12, 2), 256: (12, 2), 512: (12, 1), 1024: (12, 1),
            4096: (12, 1)}
    for m, (cfg, ks) in want.items():
        st, c, k, kslice = mp.mpgemm_plan_w4a16(m, 4096, 4096, 256)
        assert (st, c, k) == (OK, cfg, ks), m
        assert kslice == 4096 // ks


def test_w4a16_plan_invariants(mp):
    """Every split covers K with equal whole 128-k slices, none empty, none
    longer than a workgroup holds, and the partial tiles fit the workspace;
    otherwise the call falls back to a kernel without a split."""
    rng = np.random.default_rng(1)
    for _ in range(3000):
        M = int(rng.integers(1, 3000))
        N = int(rng.integers(1, 20000))
        K = int(rng.integers(0, 40000)) // 32 * 32
        st, cfg, ks, kslice = mp.mpgemm_plan_w4a16(M, N, K, 256)
        assert st == OK
        if K == 0:
            assert cfg == 3 and ks == 1
            continue
        assert ks >= 1
        if ks == 1:
            assert kslice == K
            continue
        assert cfg in SLICE
        bm, bn, span = SLICE[cfg]
        assert kslice % 128 == 0 and kslice <= span
        assert (ks - 1) * kslice < K <= ks * kslice
        tiles = -(-M // bm) * -(-N // bn)
        assert tiles * ks * bm * bn <= WORKSPACE_FLOATS


def test_w4a16_plan_falls_back_when_the_workspace_is_too_small(mp):
    """A very tall call whose partial tiles exceed the workspace runs the
    K-inside-the-workgroup MFMA kernel instead (configuration 1)."""
    st, cfg, ks, kslice = mp.mpgemm_plan_w4a16(4096, 16384, 16384, 256)
    assert (st, ks) == (OK, 1) and cfg in (1, 10)
    if cfg == 10:   # the slice kernel when no split is needed at all
        assert kslice == 16384


def test_plan_w4a16_arguments(mp):
    assert mp.mpgemm_plan_w4a16(0, 8, 8, 256)[0] == INVALID
    assert mp.mpgemm_plan_w4a16(8, 8, -8, 256)[0] == INVALID
