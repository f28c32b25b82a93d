"""Seeded synthetic inputs for the mpgemm workloads.

This module is the only code the CPU oracle and the GPU path have in common:
it produces input bytes and holds none of the GEMM arithmetic. Both sides
receive exactly the same host arrays.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: draw i of a stream with
seed s is mix(s + (i + 1) * 0x9E3779B97F4A7C15), so any slice of a stream can be
produced independently. One stream per problem; A is drawn first, then B, then
the scales.

Value recipes (the workloads of the L4 multi-precision GEMM study and of the
fused-int4-gemm-sm75 README, with the distributions of their stated configs):
  int8             top byte of a draw, uniform on [-128, 127]
  packed int4      top byte of a draw is one packed byte: two independent
                   uniform signed nibbles in [-8, 7] (low nibble = even k)
  fp16 U[lo, hi)   lo + (hi - lo) * u with u = (draw >> 11) * 2^-53,
                   rounded to binary16 by numpy (round to nearest even)
  fp16 N(0, 1)     Box-Muller on two draws, rounded to binary16
  fp16 weights     0.02 * N(0, 1) the same way (inputs of the quantiser)
"""
import math

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
# shift counts as 0-d arrays: numpy shifts by a numpy scalar far more slowly
_S11, _S27, _S30, _S31, _S56 = (np.array(v, dtype=np.uint64) for v in (11, 27, 30, 31, 56))
_CHUNK = 1 << 22


def _chunks(seed: int, start: int, count: int):
    """Yield (offset, draws) for draws start .. start+count-1 in chunks; the
    yielded array is reused by the next iteration."""
    s = np.array(seed & 0xFFFFFFFFFFFFFFFF, dtype=np.uint64)
    step = min(_CHUNK, max(count, 1))
    z = np.empty(step, dtype=np.uint64)
    t = np.empty(step, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for c0 in range(0, count, _CHUNK):
            n = min(_CHUNK, count - c0)
            zz, tt = z[:n], t[:n]
            # counter i + 1 (an int64 arange is much faster than a uint64 one)
            zz.view(np.int64)[:] = np.arange(start + c0 + 1, start + c0 + 1 + n, dtype=np.int64)
            zz *= GOLDEN
            zz += s
            for mult, sh in ((_M1, _S30), (_M2, _S27)):
                np.right_shift(zz, sh, out=tt)
                zz ^= tt
                zz *= mult
            np.right_shift(zz, _S31, out=tt)
            zz ^= tt
            yield c0, zz


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream with this seed."""
    out = np.empty(count, dtype=np.uint64)
    for c0, z in _chunks(seed, start, count):
        out[c0:c0 + z.size] = z
    return out


def _top_byte(seed, start, count):
    out = np.empty(count, dtype=np.uint8)
    for c0, z in _chunks(seed, start, count):
        out[c0:c0 + z.size] = z >> _S56
    return out


def _unit_to_f16(seed, start, count, lo, hi):
    """lo + (hi - lo) * u, u uniform in [0, 1) with 53 bits, rounded to fp16."""
    out = np.empty(count, dtype=np.float16)
    for c0, z in _chunks(seed, start, count):
        u = (z >> _S11).view(np.int64).astype(np.float64) * (2.0 ** -53)
        out[c0:c0 + z.size] = lo + (hi - lo) * u
    return out


def int8_uniform(seed: int, start: int, rows: int, cols: int) -> np.ndarray:
    return _top_byte(seed, start, rows * cols).view(np.int8).reshape(rows, cols)


def int4_packed_uniform(seed: int, start: int, rows: int, k: int) -> np.ndarray:
    """rows x ceil(k/2) packed bytes; if k is odd the unused high nibble of the
    last byte is cleared."""
    nb = (k + 1) // 2
    p = _top_byte(seed, start, rows * nb).reshape(rows, nb)
    if k % 2:
        p[:, -1] &= 0x0F
    return p


def f16_uniform(seed: int, start: int, rows: int, cols: int, lo: float, hi: float) -> np.ndarray:
    return _unit_to_f16(seed, start, rows * cols, lo, hi).reshape(rows, cols)


def f16_normal(seed: int, start: int, rows: int, cols: int) -> np.ndarray:
    n = rows * cols
    r = splitmix64(seed, start, 2 * n)
    u1 = ((r[0::2] >> _S11).view(np.int64).astype(np.float64) + 1.0) * (2.0 ** -53)   # (0, 1]
    u2 = (r[1::2] >> _S11).view(np.int64).astype(np.float64) * (2.0 ** -53)           # [0, 1)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return z.astype(np.float16).reshape(rows, cols)


def f16_weights(seed: int, start: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """fp16 weights std * N(0, 1): Box-Muller on two draws, scaled in double,
    rounded to binary16 once."""
    n = rows * cols
    r = splitmix64(seed, start, 2 * n)
    u1 = ((r[0::2] >> _S11).view(np.int64).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = (r[1::2] >> _S11).view(np.int64).astype(np.float64) * (2.0 ** -53)
    z = std * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return z.astype(np.float16).reshape(rows, cols)


def draws_f16_normal(rows: int, cols: int) -> int:
    return 2 * rows * cols


# ------------------------------------------------------------------ problems

def config_seed(config_index: int, size: int) -> int:
    """Seed of one (config, size) problem: 1000 * (config + 1) + log2(size)."""
    return 1000 * (config_index + 1) + int(math.log2(size)) if size > 0 else 1000 * (config_index + 1)


def gemm_problem(precision: str, M: int, N: int, K: int, seed: int):
    """Host inputs of C = A * B^T: A is M x K, B is N x K, both row-major.

    precision: 'i8' (int8 arrays), 'i4' (packed uint8 arrays, K/2 bytes per
    row) or 'f16' (float16 arrays, U[-1, 1)).
    """
    if precision == "i8":
        A = int8_uniform(seed, 0, M, K)
        B = int8_uniform(seed, M * K, N, K)
    elif precision == "i4":
        nb = (K + 1) // 2
        A = int4_packed_uniform(seed, 0, M, K)
        B = int4_packed_uniform(seed, M * nb, N, K)
    elif precision == "f16":
        A = f16_uniform(seed, 0, M, K, -1.0, 1.0)
        B = f16_uniform(seed, M * K, N, K, -1.0, 1.0)
    else:
        raise ValueError(precision)
    return A, B


def w4a16_problem(M: int, N: int, K: int, G: int, seed: int):
    """Activations X (M x K fp16, N(0,1)), packed INT4 weights W (N x K/2 bytes,
    uniform [-8, 7]) and scales S (N x K/G fp16, U[0.005, 0.02))."""
    X = f16_normal(seed, 0, M, K)
    off = draws_f16_normal(M, K)
    W = int4_packed_uniform(seed, off, N, K)
    off += N * ((K + 1) // 2)
    S = f16_uniform(seed, off, N, K // G, 0.005, 0.02)
    return X, W, S


def w4a4_problem(M: int, N: int, K: int, seed: int):
    """Packed INT4 activations A (M x K/2) and weights B (N x K/2), uniform
    [-8, 7]; fp16 per-row activation scales SX U[0.005, 0.02), per-row weight
    scales SW U[0.001, 0.01), column bias 0.1 * N(0, 1)."""
    nb = (K + 1) // 2
    A = int4_packed_uniform(seed, 0, M, K)
    B = int4_packed_uniform(seed, M * nb, N, K)
    off = (M + N) * nb
    SX = f16_uniform(seed, off, 1, M, 0.005, 0.02).reshape(M)
    SW = f16_uniform(seed, off + M, 1, N, 0.001, 0.01).reshape(N)
    bias = f16_weights(seed, off + M + N, 1, N, 0.1).reshape(N)
    return A, B, SX, SW, bias


def w4a4_lowrank_problem(M: int, N: int, K: int, R: int, seed: int):
    """The W4A4 problem of w4a4_problem plus the low-rank branch's inputs:
    unquantised activations X (M x K fp16, N(0, 1)), down-projection LD
    (R x K, 0.02 * N(0, 1)) and up-projection LU (N x R, 0.02 * N(0, 1)),
    drawn from the same seed after the W4A4 inputs' draws (X is drawn on its
    own, not the activations that A encodes)."""
    A, B, SX, SW, bias = w4a4_problem(M, N, K, seed)
    off = (M + N) * ((K + 1) // 2) + M + N + 2 * N
    X = f16_normal(seed, off, M, K)
    off += draws_f16_normal(M, K)
    LD = f16_weights(seed, off, R, K)
    off += 2 * R * K
    LU = f16_weights(seed, off, N, R)
    return A, B, SX, SW, bias, X, LD, LU
