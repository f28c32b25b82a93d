"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something it does not compute: a library
routine that reduces to the same mathematics (numpy's exact int64 matmul and
its IEEE binary16 conversions), exact rational arithmetic, closed forms,
invariants, or hand-worked fixtures under tests/golden/. Sources of each
definition are in oracle/oracle.h.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
# (independent of the oracle: written against the format definition)

def unpack_i4(packed: np.ndarray, K: int) -> np.ndarray:
    """Packed signed INT4 rows -> int8 rows, with numpy bit operations."""
    lo = (packed & 0x0F).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out[:, :K].astype(np.int8)


def pack_i4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape[1] % 2 == 0 and q.min() >= -8 and q.max() <= 7
    u = (q & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def rng(seed):
    return np.random.default_rng(seed)


def rand_f16(r, shape, lo=-1.0, hi=1.0):
    return r.uniform(lo, hi, size=shape).astype(np.float16)


def read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append(vals)
    return rows


# ----------------------------------------------------------------- binary16

def test_f16_decode_all_patterns_match_numpy(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.f16_decode(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(oracle_lib.f16_decode(0x8000)) and not np.signbit(oracle_lib.f16_decode(0))


def _check_encode(oracle_lib, xs):
    xs = np.asarray(xs, dtype=np.float64)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = oracle_lib.f16_encode_rne_array(xs)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_f16_encode_exact_values_and_ties(oracle_lib):
    bits = np.arange(0, 0x7C00, dtype=np.uint16)          # all finite positives
    v = bits.view(np.float16).astype(np.float64)
    _check_encode(oracle_lib, np.concatenate([v, -v]))
    # midpoints between neighbours are exact ties: round half to even
    mid = (v[:-1] + v[1:]) / 2.0
    _check_encode(oracle_lib, np.concatenate([mid, -mid]))
    # just above / below each midpoint
    _check_encode(oracle_lib, np.nextafter(mid, np.inf))
    _check_encode(oracle_lib, np.nextafter(mid, -np.inf))


def test_f16_encode_random_and_edges(oracle_lib):
    r = rng(1)
    xs = np.concatenate([
        r.uniform(-70000, 70000, 4000),
        r.standard_normal(4000),
        r.standard_normal(4000) * 2.0 ** -16,               # subnormal range
        [65504.0, 65519.99, 65520.0, 65536.0, 1e9, -65520.0, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0],
    ])
    _check_encode(oracle_lib, xs)
    assert oracle_lib.f16_encode_rne(float("inf")) == 0x7C00
    assert oracle_lib.f16_encode_rne(float("-inf")) == 0xFC00
    assert (oracle_lib.f16_encode_rne(float("nan")) & 0x7C00) == 0x7C00


# ----------------------------------------------------------------- int4 format

def test_i4_nibbles_golden(oracle_lib):
    rows = read_golden("int4_nibbles.txt")
    assert rows
    for key, vals in rows.items():
        byte = int(key, 16)
        even, odd = int(vals[0][0]), int(vals[0][1])
        row = np.array([byte], dtype=np.uint8)
        assert oracle_lib.i4_get(row, 0) == even, hex(byte)
        assert oracle_lib.i4_get(row, 1) == odd, hex(byte)


def test_i4_get_all_bytes_matches_numpy_unpack(oracle_lib):
    row = np.arange(256, dtype=np.uint8)
    ref = unpack_i4(row[None, :], 512)[0]
    got = np.array([oracle_lib.i4_get(row, k) for k in range(512)])
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------- int8 GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (4, 4, 4), (7, 13, 33), (64, 48, 100), (3, 130, 257)])
def test_i8_matches_exact_int64_matmul(oracle_lib, M, N, K):
    r = rng(M * 1000 + N * 10 + K)
    A = r.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    B = r.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    ref = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(oracle_lib.gemm_i8(A, B), ref.astype(np.int32))


def test_i8_brute_force_4x4(oracle_lib):
    A = np.array([[1, -2, 3, 127], [-128, 0, 5, 9], [4, 4, -4, 4], [0, 1, 0, -1]], dtype=np.int8)
    B = np.array([[2, 3, -1, 1], [-128, 127, 0, 2], [1, 1, 1, 1], [7, -7, 7, -7]], dtype=np.int8)
    C = oracle_lib.gemm_i8(A, B)
    # each entry written out by hand: C[i][j] = sum_k A[i][k] * B[j][k]
    assert C[0, 0] == 1 * 2 + (-2) * 3 + 3 * (-1) + 127 * 1
    assert C[0, 1] == 1 * (-128) + (-2) * 127 + 3 * 0 + 127 * 2
    assert C[1, 0] == (-128) * 2 + 0 * 3 + 5 * (-1) + 9 * 1
    assert C[1, 1] == (-128) * (-128) + 0 * 127 + 5 * 0 + 9 * 2
    assert C[2, 3] == 4 * 7 + 4 * (-7) + (-4) * 7 + 4 * (-7)
    assert C[3, 2] == 0 * 1 + 1 * 1 + 0 * 1 + (-1) * 1
    assert C[3, 3] == 0 * 7 + 1 * (-7) + 0 * 7 + (-1) * (-7)


def test_i8_identity_and_ones(oracle_lib):
    r = rng(7)
    K = 37
    A = r.integers(-128, 128, (5, K)).astype(np.int8)
    eye = np.eye(K, dtype=np.int8)
    assert np.array_equal(oracle_lib.gemm_i8(A, eye), A.astype(np.int32))          # B = I -> C = A
    assert np.array_equal(oracle_lib.gemm_i8(eye, A), A.T.astype(np.int32))        # A = I -> C = B^T
    ones_a = np.ones((3, K), dtype=np.int8)
    C = oracle_lib.gemm_i8(ones_a, A)                                               # row sums of B
    assert np.array_equal(C, np.tile(A.astype(np.int64).sum(1), (3, 1)))
    full = np.full((2, 8192), -128, dtype=np.int8)
    assert np.all(oracle_lib.gemm_i8(full, full) == 16384 * 8192)                   # 2^27


def test_i8_overflow_is_reported(oracle_lib):
    K = 131072                                  # 16384 * K = 2^31 leaves int32
    full = np.full((1, K), -128, dtype=np.int8)
    with pytest.raises(ValueError):
        oracle_lib.gemm_i8(full, full)
    ok = np.full((1, K - 1), -128, dtype=np.int8)
    assert oracle_lib.gemm_i8(ok, ok)[0, 0] == 16384 * (K - 1)


def test_i8_degenerate_shapes(oracle_lib):
    A = np.zeros((0, 5), dtype=np.int8)
    B = np.ones((3, 5), dtype=np.int8)
    assert oracle_lib.gemm_i8(A, B).shape == (0, 3)
    A0 = np.ones((2, 0), dtype=np.int8)
    B0 = np.ones((3, 0), dtype=np.int8)
    assert np.array_equal(oracle_lib.gemm_i8(A0, B0), np.zeros((2, 3), np.int32))   # K = 0 -> zeros


# ----------------------------------------------------------------- int4 GEMM

def test_i4_golden_worked_example(oracle_lib):
    g = read_golden("i4_gemm_2x2x4.txt")
    K = int(g["K"][0][0])
    A = np.array([[int(v, 16) for v in row] for row in g["A"]], dtype=np.uint8)
    B = np.array([[int(v, 16) for v in row] for row in g["B"]], dtype=np.uint8)
    C = np.array([[int(v) for v in row] for row in g["C"]], dtype=np.int32)
    assert np.array_equal(oracle_lib.gemm_i4(A, B, K), C)


@pytest.mark.parametrize("M,N,K", [(1, 1, 2), (4, 4, 4), (9, 5, 66), (33, 17, 258), (2, 70, 1024)])
def test_i4_equals_i8_of_unpacked(oracle_lib, M, N, K):
    r = rng(M + 100 * N + K)
    Ap = r.integers(0, 256, (M, K // 2), dtype=np.int64).astype(np.uint8)
    Bp = r.integers(0, 256, (N, K // 2), dtype=np.int64).astype(np.uint8)
    Au, Bu = unpack_i4(Ap, K), unpack_i4(Bp, K)
    got = oracle_lib.gemm_i4(Ap, Bp, K)
    assert np.array_equal(got, oracle_lib.gemm_i8(Au, Bu))
    assert np.array_equal(got, (Au.astype(np.int64) @ Bu.astype(np.int64).T).astype(np.int32))


def test_i4_closed_forms(oracle_lib):
    K = 8192
    m8 = pack_i4(np.full((2, K), -8))
    p7 = pack_i4(np.full((3, K), 7))
    assert np.all(oracle_lib.gemm_i4(m8, m8, K) == 64 * K)
    assert np.all(oracle_lib.gemm_i4(m8, p7, K) == -56 * K)
    # identity: B = I (N = K) -> C = A
    Kc = 16
    r = rng(3)
    q = r.integers(-8, 8, (3, Kc))
    eye = pack_i4(np.eye(Kc, dtype=np.int64))
    assert np.array_equal(oracle_lib.gemm_i4(pack_i4(q), eye, Kc), q.astype(np.int32))
    # only one nibble of a byte set: catches a swapped nibble order
    a = pack_i4(np.array([[0, 1]]))       # element k = 1 is 1
    b = pack_i4(np.array([[5, 3]]))
    assert oracle_lib.gemm_i4(a, b, 2)[0, 0] == 3


def test_i4_odd_ld_rejected(oracle_lib):
    import ctypes
    L = oracle_lib.lib()
    A = np.zeros((1, 2), dtype=np.uint8)
    C = np.zeros((1, 1), dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.oracle_gemm_i4(1, 1, 3, p(A), 3, p(A), 4, p(C), 1) == oracle_lib.ERR_ARG


# ----------------------------------------------------------------- fp16 GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (4, 4, 4), (6, 11, 129), (32, 40, 512), (3, 5, 8192)])
def test_f16_matches_exact_fixed_point(oracle_lib, M, N, K):
    """Inputs in [-1, 1] are integer multiples of 2^-24, so the exact C is an
    integer multiple of 2^-48 and numpy's int64 matmul computes it exactly
    (|sum| <= K * 2^48 < 2^63). The fp64 oracle must sit within the sequential
    summation bound K * 2^-53 * sum|a b| of it."""
    r = rng(K + 7 * M + 3 * N)
    A = rand_f16(r, (M, K))
    B = rand_f16(r, (N, K))
    Ai = (A.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    Bi = (B.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(Ai.astype(np.float64) * 2.0 ** -24, A.astype(np.float64))
    exact = Ai @ Bi.T                                            # units of 2^-48
    absum = np.abs(Ai) @ np.abs(Bi).T
    got = oracle_lib.gemm_f16(A, B)
    err = np.abs(got * 2.0 ** 48 - exact.astype(np.float64))
    bound = K * 2.0 ** -53 * absum.astype(np.float64) + 1.0
    assert np.all(err <= bound)


def test_f16_small_integers_equal_int8_oracle(oracle_lib):
    r = rng(11)
    K = 300
    A = r.integers(-4, 5, (9, K))
    B = r.integers(-4, 5, (12, K))
    got = oracle_lib.gemm_f16(A.astype(np.float16), B.astype(np.float16))
    ref = oracle_lib.gemm_i8(A.astype(np.int8), B.astype(np.int8))
    assert np.array_equal(got, ref.astype(np.float64))


def test_f16_brute_force_4x4_fractions(oracle_lib):
    r = rng(5)
    A = rand_f16(r, (4, 4), -2, 2)
    B = rand_f16(r, (4, 4), -2, 2)
    got = oracle_lib.gemm_f16(A, B)
    for i in range(4):
        for j in range(4):
            exact = sum(Fraction(float(A[i, k])) * Fraction(float(B[j, k])) for k in range(4))
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(1, 2 ** 45)


def test_f16_identity_and_transpose(oracle_lib):
    r = rng(9)
    K = 24
    A = rand_f16(r, (5, K), -100, 100)
    eye = np.eye(K, dtype=np.float16)
    assert np.array_equal(oracle_lib.gemm_f16(A, eye), A.astype(np.float64))
    assert np.array_equal(oracle_lib.gemm_f16(eye, A), A.astype(np.float64).T)
    # subnormal and infinite inputs take their IEEE values
    sub = np.array([[np.float16(2.0 ** -24)]], dtype=np.float16)
    assert oracle_lib.gemm_f16(sub, np.array([[1.0]], np.float16))[0, 0] == 2.0 ** -24
    inf = np.array([[np.inf, 1.0]], dtype=np.float16)
    assert oracle_lib.gemm_f16(inf, np.array([[1.0, 1.0]], np.float16))[0, 0] == np.inf


# ----------------------------------------------------------------- W4A16

def test_w4a16_golden_worked_example(oracle_lib):
    g = read_golden("w4a16_1x1x4.txt")
    K, G = int(g["K"][0][0]), int(g["G"][0][0])
    X = np.array([[int(v, 16) for v in g["X"][0]]], dtype=np.uint16)
    W = np.array([[int(v, 16) for v in g["W"][0]]], dtype=np.uint8)
    S = np.array([[int(v, 16) for v in g["S"][0]]], dtype=np.uint16)
    Y = oracle_lib.gemm_w4a16(X, W, S, K, G)
    assert Y[0, 0] == float(g["Y"][0][0])
    assert oracle_lib.f16_encode_rne(Y[0, 0]) == int(g["YBITS"][0][0], 16)


def _w4a16_case(seed, M, N, K, G):
    r = rng(seed)
    X = r.standard_normal((M, K)).astype(np.float16)
    Wp = r.integers(0, 256, (N, K // 2), dtype=np.int64).astype(np.uint8)
    S = r.uniform(0.005, 0.02, (N, K // G)).astype(np.float16)
    return X, Wp, S


def test_w4a16_exact_rational_small(oracle_lib):
    M, N, K, G = 2, 3, 16, 4
    X, Wp, S = _w4a16_case(21, M, N, K, G)
    q = unpack_i4(Wp, K)
    Y, T2 = oracle_lib.gemm_w4a16(X, Wp, S, K, G, want_t2=True)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(X[m, k])) * int(q[n, k]) * Fraction(float(S[n, k // G]))
                     for k in range(K)]
            exact = sum(terms)
            assert abs(Fraction(Y[m, n]) - exact) <= Fraction(1, 2 ** 40)
            assert abs(Fraction(T2[m, n]) - sum(t * t for t in terms)) <= Fraction(1, 2 ** 40)


def test_w4a16_one_hot_selects_group_and_nibble(oracle_lib):
    N, K, G = 5, 64, 8
    _, Wp, S = _w4a16_case(22, 1, N, K, G)
    S = np.arange(1, N * (K // G) + 1, dtype=np.float64).reshape(N, K // G).astype(np.float16)
    q = unpack_i4(Wp, K)
    # k at group boundaries and inside groups
    for k in [0, 1, G - 1, G, G + 1, 2 * G - 1, 2 * G, K - 1]:
        X = np.zeros((1, K), dtype=np.float16)
        X[0, k] = 1.0
        Y = oracle_lib.gemm_w4a16(X, Wp, S, K, G)
        ref = q[:, k].astype(np.float64) * S[:, k // G].astype(np.float64)
        assert np.array_equal(Y[0], ref), k


def test_w4a16_unit_scales_one_group_equals_f16_gemm(oracle_lib):
    M, N, K = 3, 7, 96
    X, Wp, _ = _w4a16_case(23, M, N, K, K)
    S = np.ones((N, 1), dtype=np.float16)
    q = unpack_i4(Wp, K).astype(np.float16)
    assert np.array_equal(oracle_lib.gemm_w4a16(X, Wp, S, K, K), oracle_lib.gemm_f16(X, q))


def test_w4a16_group_scale_closed_form(oracle_lib):
    N, K, G = 4, 128, 32
    X = np.ones((1, K), dtype=np.float16)
    Wp = pack_i4(np.ones((N, K), dtype=np.int64))
    S = (rng(24).integers(1, 64, (N, K // G)) / 64.0).astype(np.float16)
    Y = oracle_lib.gemm_w4a16(X, Wp, S, K, G)
    assert np.array_equal(Y[0], G * S.astype(np.float64).sum(1))


def test_w4a16_bad_group_rejected(oracle_lib):
    X, Wp, S = _w4a16_case(25, 1, 2, 16, 4)
    with pytest.raises(ValueError):
        oracle_lib.gemm_w4a16(X, Wp, S, 16, 5)           # K % G != 0


# ------------------------------------------------------------------ INT4 weight quantisation

def test_quantize_golden_worked_example(oracle_lib):
    """tests/golden/quantize_w4_1x8.txt: two groups worked out by hand."""
    f = {}
    for line in open(os.path.join(GOLDEN, "quantize_w4_1x8.txt")):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            f[key] = vals
    G = int(f["G"][0])
    W = np.array([[float(v) for v in f["w"]]], dtype=np.float16)
    Q, S = oracle_lib.quantize_w4(W, G)
    num = [int(v) for v in f["s_num"]]
    assert S.astype(np.float64).tolist() == [[num[0] / num[1], num[2] / num[3]]]
    assert Q.tolist() == [[int(v) for v in f["q_bytes"]]]


def test_quantize_exact_multiples_round_trip_exactly(oracle_lib):
    """Weights that are integer multiples of a power-of-two step whose group
    maximum is 7 steps: the scale is the step itself and the codes are the
    integers."""
    rng = np.random.default_rng(3)
    G, N = 32, 6
    step = 2.0 ** -rng.integers(2, 10, N)
    q = rng.integers(-7, 8, (N, 4 * G))
    q[:, ::G] = 7                      # every group reaches +7 steps
    W = (q * step[:, None]).astype(np.float16)
    Q, S = oracle_lib.quantize_w4(W, G)
    assert np.array_equal(S.astype(np.float64), np.repeat(step[:, None], 4, axis=1))
    assert np.array_equal(unpack_i4(Q, 4 * G), q)


def test_quantize_ties_round_to_even(oracle_lib):
    """w / s exactly k + 1/2 rounds to the even integer; -8 is reachable only
    through clamping, never through the symmetric scale."""
    s = 2.0 ** -4
    row = np.array([7, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5], dtype=np.float64) * s
    W = np.tile(row, (1, 4)).astype(np.float16)     # G = 32: one group of 32
    Q, S = oracle_lib.quantize_w4(W, 32)
    assert float(S[0, 0]) == s
    assert unpack_i4(Q, 32)[0, :8].tolist() == [7, 2, 4, -2, -4, 0, 0, 2]


def test_quantize_zero_group_and_bound(oracle_lib):
    """An all-zero group has scale 0 and codes 0; elsewhere every weight is
    within half a step of its dequantised value, and the group maximum maps to
    +-7."""
    rng = np.random.default_rng(11)
    N, K, G = 8, 256, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[3, 64:128] = 0
    Q, S = oracle_lib.quantize_w4(W, G)
    q = unpack_i4(Q, K)
    s = np.repeat(S.astype(np.float64), G, axis=1)
    assert S[3, 1] == 0 and np.all(q[3, 64:128] == 0)
    w = W.astype(np.float64)
    live = s > 0
    assert np.all(np.abs(w - q * s)[live] <= s[live] / 2)
    assert np.all(np.abs(q) <= 7)
    for n in range(N):
        for g in range(K // G):
            grp = w[n, g * G:(g + 1) * G]
            if np.any(grp != 0):
                i = np.argmax(np.abs(grp))
                assert abs(q[n, g * G + i]) == 7


def test_quantize_then_w4a16_one_hot_returns_dequantised_weight(oracle_lib):
    """Quantiser and weight-only GEMM share the packed layout: x = e_k gives
    y[n] = q(n, k) * s(n, k / G)."""
    rng = np.random.default_rng(5)
    N, K, G = 12, 128, 32
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    Q, S = oracle_lib.quantize_w4(W, G)
    q = unpack_i4(Q, K)
    for k in (0, 1, 31, 32, 127):
        X = np.zeros((1, K), dtype=np.float16)
        X[0, k] = 1
        y = oracle_lib.gemm_w4a16(X, Q, S, K, G)
        assert np.array_equal(y[0], q[:, k] * S[:, k // G].astype(np.float64))


def test_quantize_bad_arguments(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.quantize_w4(np.zeros((2, 96), np.float16), 64)    # K % G != 0


# ------------------------------------------------------------------ W4A4: INT4 x INT4 with scale epilogue

def _pack(q):
    q = np.asarray(q, dtype=np.int64) & 0xF
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def test_w4a4_hand_worked_2x2(oracle_lib):
    """qa = [[1, -2, 3, -8], [7, 0, -1, 2]], qb = [[2, 2, -1, 1], [-3, 4, 0, 5]]:
    row0.col0 = 2 - 4 - 3 - 8 = -13; row0.col1 = -3 - 8 + 0 - 40 = -51;
    row1.col0 = 14 + 0 + 1 + 2 = 17; row1.col1 = -21 + 0 + 0 + 10 = -11.
    SX = [0.5, 2], SW = [0.25, -1], BIAS = [1, -0.5]:
    Y = [[-13*0.125 + 1, -51*-0.5 - 0.5], [17*0.5 + 1, -11*-2 - 0.5]]
      = [[-0.625, 25.0], [9.5, 21.5]]."""
    qa = [[1, -2, 3, -8], [7, 0, -1, 2]]
    qb = [[2, 2, -1, 1], [-3, 4, 0, 5]]
    sx = np.array([0.5, 2], np.float16)
    sw = np.array([0.25, -1], np.float16)
    b = np.array([1, -0.5], np.float16)
    y = oracle_lib.gemm_w4a4(_pack(qa), _pack(qb), 4, sx, sw, b)
    assert y.tolist() == [[-0.625, 25.0], [9.5, 21.5]]


def test_w4a4_unit_scales_equal_int4_gemm(oracle_lib):
    """SX = SW = 1 and no bias: the exact INT4 product, element for element."""
    from precision_dense_gemm_tiled_amd import inputs
    M, N, K = 9, 13, 70
    Ap, Bp = inputs.gemm_problem("i4", M, N, K, seed=12)
    y = oracle_lib.gemm_w4a4(Ap, Bp, K, np.ones(M, np.float16), np.ones(N, np.float16))
    assert np.array_equal(y, oracle_lib.gemm_i4(Ap, Bp, K).astype(np.float64))


def test_w4a4_scales_and_bias_are_outer_product_and_column_shift(oracle_lib):
    """Power-of-two scales multiply exactly: Y = C * sx[m] * sw[n] + b[n]
    against the integer product C from the unit-scale call."""
    from precision_dense_gemm_tiled_amd import inputs
    M, N, K = 7, 11, 64
    Ap, Bp = inputs.gemm_problem("i4", M, N, K, seed=21)
    rng = np.random.default_rng(4)
    sx = (2.0 ** rng.integers(-6, 3, M)).astype(np.float16)
    sw = (-(2.0 ** rng.integers(-6, 3, N))).astype(np.float16)
    b = rng.integers(-8, 8, N).astype(np.float16)
    c = oracle_lib.gemm_w4a4(Ap, Bp, K, np.ones(M, np.float16), np.ones(N, np.float16))
    y = oracle_lib.gemm_w4a4(Ap, Bp, K, sx, sw, b)
    want = c * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] + b.astype(np.float64)[None, :]
    assert np.array_equal(y, want)


# ------------------------------------------------------------------ W4A4 low-rank branch L(X)

def test_w4a4_lowrank_golden_worked_example(oracle_lib):
    """The whole W4A4 formula with its low-rank branch on the hand-worked
    fixture: U, L and the fp16 output."""
    g = read_golden("w4a4_lowrank_1x2.txt")
    K = int(g["K"][0][0])

    def f(rows):
        return np.array([[float(v) for v in r] for r in rows])

    qa = [[int(v) for v in g["QA"][0]]]
    qb = [[int(v) for v in r] for r in g["QB"]]
    sx, sw, b = (f(g[k])[0].astype(np.float16) for k in ("SX", "SW", "BIAS"))
    X, LD, LU = (f(g[k]).astype(np.float16) for k in ("X", "LD", "LU"))
    U, L = oracle_lib.w4a4_lowrank(X, LD, LU)
    assert U.tolist() == f(g["U"]).tolist() and L.tolist() == f(g["L"]).tolist()
    y = oracle_lib.gemm_w4a4(_pack(qa), _pack(qb), K, sx, sw, b) + L
    assert y.tolist() == f(g["Y"]).tolist()
    assert [oracle_lib.f16_encode_rne(v) for v in y[0]] == [int(v, 16) for v in g["YBITS"][0]]


def test_w4a4_lowrank_rounds_u_to_fp16_nearest_even(oracle_lib):
    """U enters the up-projection rounded to fp16: U = 1 + 2^-10 + 2^-11 lies
    halfway between 1 + 2^-10 (odd significand) and 1 + 2^-9 (even), so it
    becomes 1 + 2^-9; U = (1 + 2^-10)^2 = 1 + 2^-9 + 2^-20 rounds down to
    1 + 2^-9; an unrounded U would give other values."""
    X = np.array([[1, 1]], np.float16)
    LD = np.array([[1 + 2 ** -10, 2 ** -11]], np.float16)
    U, L = oracle_lib.w4a4_lowrank(X, LD, np.array([[1], [-2]], np.float16))
    assert U[0, 0] == 1 + 2 ** -10 + 2 ** -11
    assert L.tolist() == [[1 + 2 ** -9, -2 - 2 ** -8]]
    X = np.array([[1 + 2 ** -10]], np.float16)
    U, L = oracle_lib.w4a4_lowrank(X, X, np.array([[1]], np.float16))
    assert U[0, 0] == 1 + 2 ** -9 + 2 ** -20 and L[0, 0] == 1 + 2 ** -9


def test_w4a4_lowrank_brute_force_rationals(oracle_lib):
    """Tiny random cases against a pure-Python evaluation in exact rationals
    (fractions), with the fp16 rounding of U done by numpy."""
    from fractions import Fraction
    r = rng(31)
    for M, N, K, R in [(1, 1, 1, 1), (2, 3, 5, 2), (3, 2, 7, 4), (4, 5, 3, 3)]:
        X = rand_f16(r, (M, K), -2, 2)
        LD = rand_f16(r, (R, K), -1, 1)
        LU = rand_f16(r, (N, R), -1, 1)
        U, L = oracle_lib.w4a4_lowrank(X, LD, LU)
        for m in range(M):
            for q in range(R):
                u = sum(Fraction(float(X[m, k])) * Fraction(float(LD[q, k])) for k in range(K))
                assert abs(Fraction(U[m, q]) - u) <= abs(u) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
            for n in range(N):
                want = sum(Fraction(float(np.float16(U[m, q]))) * Fraction(float(LU[n, q])) for q in range(R))
                assert Fraction(L[m, n]) == want


def test_w4a4_lowrank_closed_forms(oracle_lib):
    """A one-hot down-projection picks input columns (U = X[:, c], exact), so
    L = X[:, c] times the up-projection: a sum of outer products; a zero
    up-projection gives L = 0; each row of L depends only on its row of X."""
    r = rng(32)
    M, N, K, R = 6, 9, 40, 3
    X = rand_f16(r, (M, K), -4, 4)
    LD = np.zeros((R, K), np.float16)
    cols = [5, 0, 39]
    for q, c in enumerate(cols):
        LD[q, c] = 1
    LU = rand_f16(r, (N, R))
    U, L = oracle_lib.w4a4_lowrank(X, LD, LU)
    assert np.array_equal(U, X[:, cols].astype(np.float64))
    assert np.allclose(L, X[:, cols].astype(np.float64) @ LU.astype(np.float64).T, rtol=0, atol=1e-12)
    _, Z = oracle_lib.w4a4_lowrank(X, rand_f16(r, (R, K)), np.zeros((N, R), np.float16))
    assert not np.any(Z)
    X2 = X.copy()
    X2[2] = rand_f16(r, (K,))
    _, L2 = oracle_lib.w4a4_lowrank(X2, LD, LU)
    assert np.array_equal(np.delete(L2, 2, 0), np.delete(L, 2, 0)) and not np.array_equal(L2[2], L[2])
