"""The oracle pins have teeth: plausible mistakes planted in copies of
oracle.c (a dropped term, a wrong index or sign, swapped nibbles, a wrong
rounding mode, a wrong group or scale) must each fail at least one test in
test_oracle_pins.py. Each mutant is a textual change of the oracle source,
compiled like the oracle itself and loaded by the pins through
MPGEMM_ORACLE_LIB in a separate pytest process. Every mutant reads only
inside its buffers. The unmutated copy, built the same way, must pass.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")

# (name, exact fragment of oracle.c, replacement, which occurrence (0-based))
MUTANTS = [
    ("i8 drops the last k term",
     "for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)A[m * lda + k]",
     "for (int64_t k = 0; k < K - 1; ++k)\n                acc += (int64_t)A[m * lda + k]", 0),
    ("i8 pairs A[k] with B[K-1-k]",
     "(int64_t)B[n * ldb + k]", "(int64_t)B[n * ldb + (K - 1 - k)]", 0),
    ("i8 uses A's row for B",
     "(int64_t)B[n * ldb + k]", "(int64_t)A[(n < M ? n : 0) * lda + k]", 0),
    ("i8 loses the overflow report",
     "if (acc > INT32_MAX || acc < INT32_MIN)\n                overflow = 1;\n            C[m * ldc + n] = (int32_t)(uint32_t)acc;\n        }\n    }\n    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;\n}\n\nint oracle_gemm_i4",
     "(void)0;\n            C[m * ldc + n] = (int32_t)(uint32_t)acc;\n        }\n    }\n    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;\n}\n\nint oracle_gemm_i4", 0),
    ("int4 nibble order swapped",
     "(k % 2 == 0) ? (byte & 0xF) : ((byte >> 4) & 0xF)",
     "(k % 2 == 1) ? (byte & 0xF) : ((byte >> 4) & 0xF)", 0),
    ("int4 not sign-extended",
     "return (v >= 8) ? v - 16 : v;", "return v;", 0),
    ("int4 sign threshold off by one",
     "return (v >= 8) ? v - 16 : v;", "return (v > 8) ? v - 16 : v;", 0),
    ("binary16 subnormals scaled by 2^-25",
     "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 0),
    ("binary16 exponent bias off by one",
     "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);", 0),
    ("binary16 sign dropped",
     "return s ? -v : v;", "return v;", 0),
    ("binary16 encode rounds ties away from zero",
     "double q = nearbyint(ldexp(a, 10 - e));", "double q = round(ldexp(a, 10 - e));", 0),
    ("binary16 encode: subnormal ties away from zero",
     "double q = nearbyint(ldexp(a, 24));", "double q = round(ldexp(a, 24));", 0),
    ("f16 GEMM pairs a[k] with b[K-1-k]",
     "acc += a[m * K + k] * b[n * K + k];", "acc += a[m * K + k] * b[n * K + (K - 1 - k)];", 0),
    ("f16 GEMM drops the first k term",
     "double acc = 0.0;\n            for (int64_t k = 0; k < K; ++k)\n                acc += a[m * K + k]",
     "double acc = 0.0;\n            for (int64_t k = 1; k < K; ++k)\n                acc += a[m * K + k]", 0),
    ("w4a16 scale of the next group",
     "S[n * lds + k / G]", "S[n * lds + (k / G + 1) % (K / G)]", 0),
    ("w4a16 scales of row 0 for every row",
     "S[n * lds + k / G]", "S[k / G]", 0),
    ("w4a16 activations of row 0 for every row",
     "double t = x[m * K + k]", "double t = x[k]", 0),
    ("w4a16 scale applied twice",
     "* (double)oracle_i4_get(wrow, k) * s;", "* (double)oracle_i4_get(wrow, k) * s * s;", 0),
    ("w4a4 bias dropped",
     "y += oracle_f16_decode(BIAS[n]);", "y += 0.0;", 0),
    ("w4a4 row factor of row 0",
     "const double sx = oracle_f16_decode(SX[m]);", "const double sx = oracle_f16_decode(SX[0]);", 0),
    ("w4a4 column factor of column 0",
     "double y = (double)acc * sx * oracle_f16_decode(SW[n]);",
     "double y = (double)acc * sx * oracle_f16_decode(SW[0]);", 0),
    ("low-rank U not rounded to fp16",
     "l += oracle_f16_decode(oracle_f16_encode_rne(U[m * ldU + r])) * oracle_f16_decode(LU[n * ldu + r]);",
     "l += U[m * ldU + r] * oracle_f16_decode(LU[n * ldu + r]);", 0),
    ("low-rank down-projection row 0 for every r",
     "* oracle_f16_decode(LD[r * ldd + k]);", "* oracle_f16_decode(LD[k]);", 0),
    ("low-rank up-projection column 0 for every r",
     "* oracle_f16_decode(LU[n * ldu + r]);", "* oracle_f16_decode(LU[n * ldu]);", 0),
    ("low-rank drops the last k term",
     "for (int64_t k = 0; k < K; ++k)\n                u += ", "for (int64_t k = 0; k < K - 1; ++k)\n                u += ", 0),
    ("quantiser scale amax / 8",
     "oracle_f16_encode_rne(amax / 7.0)", "oracle_f16_encode_rne(amax / 8.0)", 0),
    ("quantiser rounds ties away from zero",
     "double r = nearbyint(oracle_f16_decode(W[n * ldw + k]) / s);",
     "double r = round(oracle_f16_decode(W[n * ldw + k]) / s);", 0),
    ("quantiser truncates",
     "double r = nearbyint(oracle_f16_decode(W[n * ldw + k]) / s);",
     "double r = trunc(oracle_f16_decode(W[n * ldw + k]) / s);", 0),
    ("quantiser clamps at 6",
     "q = r > 7.0 ? 7 : (r < -8.0 ? -8 : (int)r);", "q = r > 6.0 ? 6 : (r < -8.0 ? -8 : (int)r);", 0),
    ("quantiser nibble order swapped",
     "qrow[k / 2] |= (uint8_t)((k % 2) ? (nib << 4) : nib);",
     "qrow[k / 2] |= (uint8_t)((k % 2) ? nib : (nib << 4));", 0),
    ("quantiser amax over the first half of the group",
     "for (int64_t k = g * G; k < (g + 1) * G; ++k) {\n                double a = fabs",
     "for (int64_t k = g * G; k < g * G + G / 2; ++k) {\n                double a = fabs", 0),
]


def _replace_nth(text, old, new, nth):
    start = -1
    for _ in range(nth + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"fragment not found: {old!r}"
    return text[:start] + new + text[start + len(old):]


def _build(src_text, out_dir):
    os.makedirs(out_dir, exist_ok=True)
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), out_dir)
    src = os.path.join(out_dir, "oracle.c")
    with open(src, "w") as f:
        f.write(src_text)
    lib = os.path.join(out_dir, "liboracle.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", lib, src, "-lm"],
                   check=True, capture_output=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, MPGEMM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def _source():
    with open(os.path.join(ORACLE_DIR, "oracle.c")) as f:
        return f.read()


def test_unmutated_copy_passes(tmp_path):
    r = _run_pins(_build(_source(), str(tmp_path / "control")))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, nth, tmp_path):
    src = _source()
    mutated = _replace_nth(src, old, new, nth)
    assert mutated != src
    r = _run_pins(_build(mutated, str(tmp_path / "mutant")))
    assert r.returncode != 0, f"the mutant '{name}' passed every pin"
