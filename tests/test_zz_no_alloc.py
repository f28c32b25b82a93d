"""The allocation-free weight-only entry point (mpgemm_run_w4a16_noalloc),
called through the C-ABI, against the handle entry point mpgemm_run_w4a16 and
the oracle: two calls in a row that both split K into the static scratch
(the second smaller), a problem whose split needs more than the scratch
(refused, output untouched), and a call after the refusal."""
import numpy as np
import pytest

import oracle
import precision_dense_gemm_tiled_amd as mp
from precision_dense_gemm_tiled_amd import inputs
from tests.gpu_util import dev, host, require_gpu, w4a16_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu(oracle_lib):
    require_gpu()
    return True


def _noalloc(X, W, S, G, Y):
    import torch
    M, K = X.shape
    N = W.shape[0]
    return mp.mpgemm_run_w4a16_noalloc(M, N, K, X.data_ptr(), X.stride(0), W.data_ptr(), 2 * W.stride(0),
                                       S.data_ptr(), S.stride(0), G, Y.data_ptr(), Y.stride(0),
                                       torch.cuda.current_stream().cuda_stream)


def _handle(X, W, S, G, Y):
    import torch
    M, K = X.shape
    N = W.shape[0]
    return mp.mpgemm_run_w4a16(mp.default_handle(), M, N, K, X.data_ptr(), X.stride(0), W.data_ptr(),
                               2 * W.stride(0), S.data_ptr(), S.stride(0), G, Y.data_ptr(), Y.stride(0),
                               torch.cuda.current_stream().cuda_stream)


def _case(M, N, K, G, seed):
    import torch
    X, W, S = inputs.w4a16_problem(M, N, K, G, seed)
    x, w, s = dev(X), dev(W), dev(S)
    y_na = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    y_h = torch.full((M, N), -7.0, dtype=torch.float16, device="cuda")
    return (X, W, S), (x, w, s), y_na, y_h


@pytest.mark.parametrize("first,second", [((128, 4096, 4096, 128), (96, 1024, 2048, 128))])
def test_noalloc_matches_handle_entry_point_twice(first, second):
    """Both problems split K (the first over 64 x 128 slice tiles, the second
    over the ring kernel's tiles), so both go through the static scratch; the
    second call is smaller and reuses what the first left there."""
    for (M, N, K, G), seed in [(first, 31), (second, 32)]:
        st, cfg, ks, _ = mp.mpgemm_plan_w4a16(M, N, K)
        assert st == 0 and ks > 1, "the case must split K"
        (X, W, S), (x, w, s), y_na, y_h = _case(M, N, K, G, seed)
        assert _noalloc(x, w, s, G, y_na) == 0
        assert _handle(x, w, s, G, y_h) == 0
        got, want = host(y_na).view(np.uint16), host(y_h).view(np.uint16)
        assert np.array_equal(got, want), f"{M}x{N}x{K}: differs from mpgemm_run_w4a16"
        y, t2 = oracle.gemm_w4a16(X, W, S, K, G, want_t2=True)
        err = np.abs(got.view(np.float16).astype(np.float64) - y)
        assert np.all(err <= w4a16_tol(y, t2, K)), f"{M}x{N}x{K}: outside the bar"


def test_noalloc_refuses_splits_beyond_the_scratch_then_still_runs():
    """M = 128, N = K = 8192 splits K 8 ways over 64 x 128 tiles: 32 MiB of
    fp32 slices, more than the 16 MiB scratch. Refused before any launch, the
    output untouched; a following call that fits runs normally."""
    import torch
    M, N, K, G = 128, 8192, 8192, 128
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    w = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // G), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    assert _noalloc(x, w, s, G, y) == mp.MPGEMM_ERR_UNSUPPORTED
    assert torch.all(y == 3.0).item()
    # the handle entry point runs the same problem (its workspace holds it)
    assert _handle(x, w, s, G, y) == 0
    assert torch.all(y == 0.0).item()
    (X, W, S), (x, w, s), y_na, y_h = _case(16, 4096, 4096, 128, 33)
    assert _noalloc(x, w, s, 128, y_na) == 0
    assert _handle(x, w, s, 128, y_h) == 0
    assert np.array_equal(host(y_na).view(np.uint16), host(y_h).view(np.uint16))
