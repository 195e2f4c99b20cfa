"""The streaming-read measurement aid (dpsgd_hbm_read): the XOR of its sink words equals the XOR
of every 32-bit word of the buffer, computed on the host."""
import numpy as np
import pytest
import torch

import differentially_private_amd as dp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1040, 4096 * 64 + 48, 64 << 20])
def test_hbm_read_xor_matches_host(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    dev = torch.device("cuda:0")
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.full((dp.HBM_READ_SINK_WORDS,), -1, dtype=torch.int32, device=dev)
    dp.hbm_read(buf.data_ptr(), nbytes, sink.data_ptr())
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
