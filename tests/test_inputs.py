"""The seeded input generator: published SplitMix64 outputs and value ranges."""
import numpy as np

from precision_dense_gemm_tiled_amd import inputs


def test_splitmix64_reference_outputs():
    # Outputs of the published splitmix64.c reference generator.
    assert [int(v) for v in inputs.splitmix64(1234567, 0, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]
    assert int(inputs.splitmix64(0, 0, 1)[0]) == 0xE220A8397B1DCDAF


def test_splitmix64_counter_slices_agree():
    full = inputs.splitmix64(99, 0, 10000)
    assert np.array_equal(full[1234:5678], inputs.splitmix64(99, 1234, 5678 - 1234))


def test_value_recipes_ranges():
    a = inputs.int8_uniform(5, 0, 256, 256)
    assert a.dtype == np.int8 and a.min() == -128 and a.max() == 127
    assert abs(float(a.astype(np.float64).mean())) < 1.0
    p = inputs.int4_packed_uniform(5, 0, 64, 512)
    assert p.shape == (64, 256)
    nib = np.concatenate([(p & 0xF).ravel(), (p >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()
    odd = inputs.int4_packed_uniform(5, 0, 3, 7)
    assert np.all((odd[:, -1] >> 4) == 0)
    f = inputs.f16_uniform(5, 0, 128, 128, -1.0, 1.0)
    assert f.dtype == np.float16 and f.min() >= -1.0 and f.max() <= 1.0
    n = inputs.f16_normal(5, 0, 256, 256).astype(np.float64)
    assert abs(n.mean()) < 0.02 and abs(n.std() - 1.0) < 0.02
    s = inputs.f16_uniform(5, 0, 64, 32, 0.005, 0.02).astype(np.float64)
    assert s.min() >= float(np.float16(0.005)) and s.max() <= float(np.float16(0.02))


def test_problems_are_deterministic_and_distinct():
    A1, B1 = inputs.gemm_problem("i8", 64, 32, 96, inputs.config_seed(0, 512))
    A2, B2 = inputs.gemm_problem("i8", 64, 32, 96, inputs.config_seed(0, 512))
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert not np.array_equal(A1[:32], B1)
    assert inputs.config_seed(0, 512) == 1009 and inputs.config_seed(4, 1) == 5000
    X, W, S = inputs.w4a16_problem(2, 16, 256, 128, 5000)
    assert X.shape == (2, 256) and W.shape == (16, 128) and S.shape == (16, 2)
