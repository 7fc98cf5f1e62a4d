"""q8_stream_read, the on-box read-bandwidth reference: every 16-byte chunk
of the rounded-down range is read exactly once (the XOR of the per-workgroup
words equals the host's XOR of the same 32-bit words) for any grid, including
grids with more workgroups than chunks and chunks that end mid-sweep."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1000, (1 << 20) + 48, (64 << 20) + 16])
@pytest.mark.parametrize("grid", [1, 7, 4096])
def test_stream_read_xor(nbytes, grid):
    rng = np.random.default_rng(nbytes * 31 + grid)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    out = torch.full((grid + 1,), 12345, dtype=torch.int32, device="cuda")
    q.q8_stream_read(buf, out, grid)
    words = out.cpu().numpy().view(np.uint32)
    assert words[grid] == 12345  # nothing beyond the grid's words is written
    used = nbytes // 16 * 16
    want = np.bitwise_xor.reduce(host[:used].view(np.uint32)) if used else np.uint32(0)
    assert int(np.bitwise_xor.reduce(words[:grid])) == int(want)


def test_stream_read_empty_and_invalid():
    out = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    q.q8_stream_read(buf[:8], out, 4)  # under 16 bytes: nothing read, zero words
    assert out.cpu().tolist() == [0, 0, 0, 0]
    lib = q.lib()
    assert lib.q8_stream_read(buf.data_ptr(), 64, out.data_ptr(), 0, None) == q.Q8_EINVAL
    assert lib.q8_stream_read(buf.data_ptr(), 64, out.data_ptr(), -1, None) == q.Q8_EINVAL
    assert lib.q8_stream_read(buf.data_ptr() + 4, 48, out.data_ptr(), 1, None) == q.Q8_EALIGN
    with pytest.raises(ValueError):
        q.q8_stream_read(buf, out, 5)
