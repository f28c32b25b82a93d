"""The streaming-read measurement call (mpgemm_stream_read) reads every
byte: the XOR of the per-workgroup words equals numpy's XOR of the buffer,
for several sizes (a ragged last workgroup) and every loads-per-lane
setting; invalid arguments are refused."""
import numpy as np
import pytest

import precision_dense_gemm_tiled_amd as mp
from tests.gpu_util import host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()
    return True


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 * 3 + 48, 8667136])
@pytest.mark.parametrize("lpl", [1, 2, 4, 8])
def test_stream_read_xor(nbytes, lpl):
    import torch
    rng = np.random.default_rng(nbytes + lpl)
    data = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(data).cuda()
    words = -(-nbytes // (4096 * lpl))
    sink = torch.full((words + 3,), -1, dtype=torch.int32, device="cuda")
    st = mp.mpgemm_stream_read(src.data_ptr(), nbytes, lpl, sink.data_ptr(), words,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    got = np.bitwise_xor.reduce(host(sink)[:words].view(np.uint32))
    want = np.bitwise_xor.reduce(data.view(np.uint32))
    assert got == want
    assert np.all(host(sink)[words:] == -1), "wrote past the workgroup words"


def test_stream_read_argument_errors():
    import torch
    src = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert mp.mpgemm_stream_read(src.data_ptr(), 4096, 3, sink.data_ptr(), 4, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_stream_read(src.data_ptr(), 4008, 1, sink.data_ptr(), 4, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_stream_read(src.data_ptr() + 8, 4080, 1, sink.data_ptr(), 4, s) == mp.MPGEMM_ERR_UNSUPPORTED
    assert mp.mpgemm_stream_read(src.data_ptr(), 4096 * 8, 1, sink.data_ptr(), 4, s) == mp.MPGEMM_ERR_INVALID_ARG
    assert mp.mpgemm_stream_read(0, 4096, 1, sink.data_ptr(), 4, s) == mp.MPGEMM_ERR_INVALID_ARG
