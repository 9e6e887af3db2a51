"""The calibration library's streaming kernels, which set the HBM ceilings the
bench reports, do what they claim: the copy reproduces its source byte for
byte (including a length that leaves the last pass partly empty) and the read
leaves every buffer untouched."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _stream():
    from token_sparse_attention_block_amd import build as B
    f = ctypes.CDLL(B.CALIB_LIB).jano_calib_stream
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return f


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (16 * 1000 + 16 * 37, 3), (1 << 24, 64), ((1 << 24) + 4096, 4096)])
def test_stream_copy_and_read(torch, nbytes, wgs):
    print("calib stream", nbytes, wgs, flush=True)
    f = _stream()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(wgs * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert f(0, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, wgs,
             ctypes.c_void_p(sink.data_ptr()), st) == 0
    assert f(1, ctypes.c_void_p(dst.data_ptr()), None, nbytes, wgs, ctypes.c_void_p(sink.data_ptr()), st) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dst.cpu().numpy(), host)
    np.testing.assert_array_equal(src.cpu().numpy(), host)
