"""The streaming-read probe reads every byte: its XOR checksum equals the
host XOR of all 32-bit words, on sizes that leave a partial last workgroup,
on both sides of the 32 MB switch from one chunk per thread (up to 8192
workgroups) to the grid-stride pass."""
import numpy as np
import pytest
import torch

from quantized_matvec_amd import qmv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 37 * 4096 * 16 + 16, (1 << 25), (1 << 25) + 16])
def test_stream_read_checksum(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = qmv.stream_read(buf)
    want = np.bitwise_xor.reduce(words)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
