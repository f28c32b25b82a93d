"""The weight quantiser's arithmetic shortcuts, checked on the CPU.

The quantiser kernel (symmetric round-to-nearest INT4 per (row, K group):
s = fp16(max|w| / 7), q = clamp(round_half_even(w / s), -8, 7), the reading
of the "fused-int4-gemm-sm75" README's per-group scales) avoids exact
arithmetic in two places:

1. the scale is fp16(fp32(amax) * fp32(1/7)): an fp32 product rounded again
   to fp16, claimed equal to rounding the exact quotient amax / 7 once;
2. the code: with r the fp32 reciprocal of s (correctly rounded, or one ulp
   off, as the hardware reciprocal), y = fma(w, r, 192) rounds w * r once to
   the 2^-16 grid of [128, 256), y is clamped to [184, 199], and
   y + (1.5 * 2^23 + 8 - 192) rounds half to even to an integer whose low
   byte is q + 8; claimed equal to clamp(round_half_even(w / s), -8, 7).

Here the fp32 steps are replayed exactly (the rounding of the fused
multiply-add with integer arithmetic on the significands, the others in
float64, where these values are exact) and compared with exact arithmetic:
float64 values of binary16 numbers and of small multiples of them are exact,
so the distances below carry no rounding. These tests pin the kernel's
method, not the oracle.
"""
import numpy as np
import pytest


def _all_positive_f16():
    """Every finite positive binary16 value, as float64 (exact)."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def _f16_neighbours(x):
    """Next binary16 values below and above each positive binary16 x."""
    b = x.astype(np.float16).view(np.uint16).astype(np.int32)
    lo = np.clip(b - 1, 0, 0x7BFF).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = np.clip(b + 1, 0, 0x7BFF).astype(np.uint16).view(np.float16).astype(np.float64)
    return lo, hi


def test_scale_rounding_over_every_binary16_amax():
    """fp16(fp32(amax) * fp32(1/7)) is the binary16 value nearest to
    amax / 7 (ties to even) for every finite positive binary16 amax."""
    amax = _all_positive_f16()
    s = (amax.astype(np.float32) * np.float32(1.0 / 7.0)).astype(np.float16).astype(np.float64)
    lo, hi = _f16_neighbours(s)
    # compare distances times 7: |amax - 7 v| is exact in float64 (7 v has
    # at most 14 significant bits, amax and 7 v are within 2^17 of each other)
    d = np.abs(amax - 7.0 * s)
    d_lo = np.abs(amax - 7.0 * lo)
    d_hi = np.abs(amax - 7.0 * hi)
    assert np.all(d <= d_lo) and np.all(d <= d_hi), "a neighbour is nearer"
    # a tie with a neighbour would have to resolve to the even significand
    # (neighbours clipped at 0 or at the largest finite value equal s itself)
    even = (s.astype(np.float16).view(np.uint16) & 1) == 0
    tie = ((d == d_lo) & (lo != s)) | ((d == d_hi) & (hi != s))
    assert np.all(even[tie]), "tie not resolved to even"
    # amax / 7 is never exactly halfway between binary16 values (7 is odd)
    assert not np.any(tie)


def _significand(x, bits):
    """x = sign * m * 2^e with m an integer below 2^bits (x finite, exact)."""
    f, e = np.frexp(np.abs(x))
    m = np.round(f * 2.0 ** bits).astype(np.int64)     # exact: x has <= bits significant bits
    return np.sign(x).astype(np.int64), m, e.astype(np.int64) - bits


def _rhe_shift(t, sh):
    """round_half_even(t * 2^sh) for non-negative int64 t and int64 sh."""
    up = np.where(sh >= 0, t << np.clip(sh, 0, 62), 0)
    n = np.clip(-sh, 1, 62)
    q0 = t >> n
    rem = t - (q0 << n)
    half = np.int64(1) << (n - 1)
    down = q0 + ((rem > half) | ((rem == half) & (q0 % 2 == 1))).astype(np.int64)
    down = np.where(-sh > 60, 0, down)                   # t < 2^35: far below one half
    return np.where(sh >= 0, up, down)


def _kernel_code(w, s, inv):
    """The kernel's code for weight w with scale s and fp32 reciprocal inv:
    y = fp32(fma(w, inv, 192)) (one rounding of the exact value to the 2^-16
    grid), clamped to [184, 199], then rounded half to even to an integer
    (the fp32 add of 1.5 * 2^23 + 8 - 192); q = that integer - 192."""
    inv = inv.astype(np.float64)
    assert np.all(np.abs(w * inv) < 64), "y must stay in [128, 256)"
    sw, mw, ew = _significand(w, 11)
    si, mi, ei = _significand(inv, 24)
    # y * 2^16 = 192 * 2^16 + round_half_even(w * inv * 2^16): adding the
    # even integer 192 * 2^16 commutes with the rounding
    r = _rhe_shift(mw * mi, ew + ei + 16) * sw * si
    y = np.clip(192 * 65536 + r, 184 * 65536, 199 * 65536)
    base, frac = y >> 16, y & 0xFFFF
    up = (frac > 0x8000) | ((frac == 0x8000) & (base % 2 == 1))
    return (base + up.astype(np.int64) - 192).astype(np.float64)


def _exact_code(w, s):
    """round_half_even(w / s) clamped to [-8, 7], decided with exact
    remainders: c = nearest integer candidate, then |w - c s| against s / 2."""
    c = np.round(w / s)                  # a candidate within one of the answer
    for _ in range(2):                   # move c to the nearest integer
        r = w - c * s
        c = np.where(2 * r > s, c + 1, np.where(2 * r < -s, c - 1, c))
    r = w - c * s
    tie = np.abs(2 * r) == s
    c = np.where(tie & (np.abs(c) % 2 == 1), c + np.sign(r), c)
    return np.clip(c, -8, 7)


def _reciprocals(s):
    """1/s correctly rounded to fp32, and one fp32 ulp below and above."""
    inv = (np.float32(1.0) / s.astype(np.float32)).astype(np.float32)
    return [inv, np.nextafter(inv, np.float32(0)), np.nextafter(inv, np.float32(np.inf))]


@pytest.mark.parametrize("which", [0, 1, 2], ids=["exact_reciprocal", "one_ulp_low", "one_ulp_high"])
def test_code_rounding_at_and_next_to_every_half_integer(which):
    """For every finite positive binary16 scale s and every half-integer h in
    [-7.5, 7.5]: w = the binary16 values at and next to h s (two neighbours
    each side), and also at and next to the integer multiples q s. The
    snapped rounding must give round_half_even(w / s) exactly."""
    s_all = _all_positive_f16()
    halves = np.arange(-15, 16, 2, dtype=np.float64) / 2.0          # -7.5 ... 7.5
    ints = np.arange(-8, 8, dtype=np.float64)
    mult = np.concatenate([halves, ints])
    mism = 0
    checked = 0
    for chunk in np.array_split(s_all, 8):
        s = np.repeat(chunk, mult.size)
        target = s * np.tile(mult, chunk.size)                       # exact
        with np.errstate(over="ignore"):
            w0 = target.astype(np.float16)                           # nearest binary16
        ok = np.isfinite(w0)
        s, w0 = s[ok], w0[ok]
        b = w0.view(np.uint16).astype(np.int32)
        cands = []
        for d in (-2, -1, 0, 1, 2):
            # step along the binary16 encoding (sign-magnitude: step the
            # magnitude bits, keep the sign)
            mag = np.clip((b & 0x7FFF) + d, 0, 0x7BFF)
            cands.append(((b & 0x8000) | mag).astype(np.uint16).view(np.float16).astype(np.float64))
        w = np.concatenate(cands)
        ss = np.tile(s, 5)
        keep = np.abs(w / ss) <= 7.5 + 1e-9
        w, ss = w[keep], ss[keep]
        inv = _reciprocals(ss)[which]
        got = _kernel_code(w, ss, inv)
        want = _exact_code(w, ss)
        mism += int(np.count_nonzero(got != want))
        checked += w.size
    assert checked > 4_000_000
    assert mism == 0, f"{mism} of {checked} codes differ from round_half_even(w / s)"


def test_code_rounding_random_pairs():
    """A seeded sample of random binary16 pairs (w, s) with |w / s| <= 7.5,
    including subnormal scales, with all three reciprocals."""
    rng = np.random.default_rng(12345)
    s = rng.integers(1, 0x7C00, 4_000_000).astype(np.uint16).view(np.float16).astype(np.float64)
    t = rng.uniform(-7.5, 7.5, s.size)
    with np.errstate(over="ignore"):
        w = (t * s).astype(np.float16).astype(np.float64)
    keep = np.isfinite(w) & (np.abs(w / s) <= 7.5)
    w, s = w[keep], s[keep]
    want = _exact_code(w, s)
    for inv in _reciprocals(s):
        assert np.array_equal(_kernel_code(w, s, inv), want)


def test_code_clamps_past_the_range():
    """Subnormal scales: fp16(amax / 7) can fall well below amax / 7, so that
    |w / s| reaches up to 10.5; the clamp of y must give clamp(rhe(w / s))."""
    rng = np.random.default_rng(7)
    s = rng.integers(1, 0x0400, 200_000).astype(np.uint16).view(np.float16).astype(np.float64)   # subnormal
    t = rng.uniform(-10.5, 10.5, s.size)
    w = (t * s).astype(np.float16).astype(np.float64)
    keep = np.abs(w / s) <= 10.5
    w, s = w[keep], s[keep]
    assert np.any(np.abs(w / s) > 8)
    want = _exact_code(w, s)
    for inv in _reciprocals(s):
        assert np.array_equal(_kernel_code(w, s, inv), want)


def test_exact_code_reference_by_hand():
    """The exact reference on hand-worked values (ties to even, clamping)."""
    s = np.full(9, 0.5)
    w = np.array([0.25, 0.75, -0.25, -0.75, 1.25, 3.74, 3.76, -4.25, 4.0])
    assert np.array_equal(_exact_code(w, s), [0, 2, 0, -2, 2, 7, 7, -8, 7])
    # and the kernel's method on the same values
    assert np.array_equal(_kernel_code(w, s, _reciprocals(s)[0]), [0, 2, 0, -2, 2, 7, 7, -8, 7])
