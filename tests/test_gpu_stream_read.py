"""q8_stream_read, the on-box read-bandwidth reference: it must read every
16-byte chunk of the rounded-down range exactly once (the XOR of all 32-bit
words read equals the host's XOR of the same words) for any grid, including
grids that leave a ragged tail of the grid-stride loop."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1000, (1 << 20) + 48, (64 << 20) + 16])
@pytest.mark.parametrize("grid", [0, 1, 7, 4096])
def test_stream_read_xor(nbytes, grid):
    rng = np.random.default_rng(nbytes * 31 + grid)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.q8_stream_read(buf, out, grid)
    torch.cuda.synchronize()
    used = nbytes // 16 * 16
    want = np.bitwise_xor.reduce(host[:used].view(np.uint32)) if used else np.uint32(0)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_stream_read_empty_and_invalid():
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    q.q8_stream_read(buf[:0], out)
    torch.cuda.synchronize()
    assert int(out.cpu()[0]) == 0
    lib = q.lib()
    assert lib.q8_stream_read(buf.data_ptr(), 64, out.data_ptr(), -1, None) == q.Q8_EINVAL
    assert lib.q8_stream_read(buf.data_ptr() + 4, 48, out.data_ptr(), 0, None) == q.Q8_EALIGN
