"""Helpers shared by the GPU tests: device transfer and the stated tolerances."""
import math

import numpy as np

# Tile configurations of the GEMM kernels (indices of the MPGEMM_TILE_CFG
# override): 0-11 the ring kernel's shapes, 12 the 256 x 256 ping-pong kernel,
# 13-17 one-change ablations of the 256 x 256 ring (split loaders, nt, sc1,
# VGPR-staged loads, spread loads), 18 the 256 x 256 kernel with B loaded
# straight into registers, 19 the sc0 cache-policy ablation of the ring, 20
# the ring with each k-step's fragment reads fenced ahead of its MFMAs.
N_TILE_CFGS = 23
PINGPONG_CFG = 12
B_DIRECT_CFGS = (18,)


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a gfx950 device (torch.cuda.is_available() is False)")
    return torch


def dev(a: np.ndarray):
    """numpy host array -> contiguous device tensor with the same bytes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16_tol(K: int) -> float:
    """FP16 bar: per-element |C_gpu - C_ref| <= 2^-10 * sqrt(K) against fp64."""
    return 2.0 ** -10 * math.sqrt(max(K, 1))


def w4a4_tol(y, c_abs, sx, sw, b):
    """W4A4 bar: fp16 output rounding (half an ulp: 2^-11 relative) plus the
    fp32 epilogue (two products and one sum, each within 2^-24 relative) plus
    subnormals; c_abs = |exact integer product|."""
    mag = c_abs * np.abs(sx.astype(np.float64))[:, None] * np.abs(sw.astype(np.float64))[None, :]
    bb = np.abs(b.astype(np.float64))[None, :] if b is not None else 0.0
    return 2.0 ** -11 * np.abs(y) + 3 * 2.0 ** -24 * (mag + bb) + 2.0 ** -24


def w4a16_tol(y_ref: np.ndarray, t2: np.ndarray, K: int) -> np.ndarray:
    """W4A16 bar: half an fp16 ulp of the output, plus fp16 dequantisation
    rounding of each term (relative 2^-11, random sign, summed over K terms of
    rms sigma_t = sqrt(T2 / K), kept at 2^-9 * sqrt(K) * sigma_t), plus 2^-24 for
    subnormal outputs."""
    sigma_t = np.sqrt(t2 / max(K, 1))
    return 2.0 ** -11 * np.abs(y_ref) + 2.0 ** -9 * math.sqrt(max(K, 1)) * sigma_t + 2.0 ** -24


def unpack_i4(packed: np.ndarray, K: int) -> np.ndarray:
    """Packed signed INT4 rows -> int8 rows (numpy bit operations, test side)."""
    lo = (packed & 0x0F).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out[:, :K].astype(np.int8)


def pack_i4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    u = (q & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def freivalds_int(C: np.ndarray, A: np.ndarray, B: np.ndarray, seed: int, trials: int = 3):
    """Exact check of C == A @ B.T over every element with random +-1 vectors
    (int64 arithmetic; an error in any single element always changes C @ r)."""
    rng = np.random.default_rng(seed)
    A64 = A.astype(np.int64)
    B64 = B.astype(np.int64)
    C64 = C.astype(np.int64)
    for _ in range(trials):
        r = rng.choice(np.array([-1, 1], dtype=np.int64), size=C.shape[1])
        lhs = C64 @ r
        rhs = A64 @ (B64.T @ r)
        bad = np.nonzero(lhs != rhs)[0]
        assert bad.size == 0, f"Freivalds mismatch in rows {bad[:8]}"


def band_rows(M: int, band: int, per_band: int) -> np.ndarray:
    """per_band rows in each band of `band` consecutive rows, at offsets
    within the band that differ from band to band (a fixed odd stride), so
    together they reach many row positions of an output tile."""
    rows = []
    for b0 in range(0, M, band):
        size = min(band, M - b0)
        for j in range(per_band):
            rows.append(b0 + ((b0 // band) * 37 + j * (size // per_band + 1)) % size)
    return np.array(sorted(set(rows)))
