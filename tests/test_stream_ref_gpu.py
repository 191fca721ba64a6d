"""The benchmark's read-only streaming reference reads every byte once: its
XOR checksum equals the host's, for sizes that do not divide the grid."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pq = pytest.importorskip("decode_attention_product_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid,block", [(16, 1, 64), (9864192, 256, 1024),
                                               (1 << 20, 2048, 256), (4096 * 16 + 48, 7, 192)])
def test_stream_read_checksum(nbytes, grid, block):
    path = os.path.join(os.path.dirname(pq.LIB_PATH), "libpqbench.so")
    lib = ctypes.CDLL(path)
    lib.pqbench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    chk = torch.zeros(grid, dtype=torch.int32, device="cuda")
    st = lib.pqbench_stream_read(buf.data_ptr(), nbytes, chk.data_ptr(), grid, block,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host)
    assert int(np.bitwise_xor.reduce(chk.cpu().numpy().view(np.uint32))) == int(expect)
