"""The benchmark's memory-ceiling probe (libconvrot_ceiling.so) on the GPU: its 2:1 pattern moves
exactly the bytes it is described to move (the high byte of every 16-bit element of X into the
tiled code layout), so the ceiling it reports is the ceiling of real work."""
import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import need_gpu, untile_codes
from w4a4_integer_quantized_amd import build as B

pytestmark = pytest.mark.gpu


def _fn():
    if not os.path.exists(B.CEILING_LIB):
        pytest.fail("libconvrot_ceiling.so is not built")
    fn = ctypes.CDLL(B.CEILING_LIB).rqc_hbm_pattern
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


@pytest.mark.parametrize("M,K", [(300, 1024), (37, 4096), (1, 128), (513, 1536)])
def test_ceiling_copy_pattern_moves_the_high_bytes(M, K):
    need_gpu()
    print("ceiling case M=%d K=%d" % (M, K), flush=True)
    rng = np.random.default_rng(M + K)
    xb = rng.integers(0, 1 << 16, (M, K), dtype=np.uint16)
    X = torch.from_numpy(xb.view(np.int16)).cuda()
    Q = torch.full((-(-M // 256) * 256 * K,), 0x5A, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert _fn()(0, X.data_ptr(), Q.data_ptr(), M, K, 1, stream) == 0
    torch.cuda.synchronize()
    got = untile_codes(Q.cpu().numpy(), M, K, 8).view(np.uint8)
    assert np.array_equal(got, (xb >> 8).astype(np.uint8))
