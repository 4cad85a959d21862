"""The streaming-read probe that gives the bench its measured HBM read
ceiling: every 32-bit word of the buffer is read exactly once, so the XOR of
the per-wave sink words equals the XOR of the buffer's words."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa

from helpers import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 4097, (64 << 20) // 16 + 3])
def test_stream_read_reads_every_word_once(n16):
    announce(f"stream_read n16={n16}")
    g = torch.Generator().manual_seed(n16)
    host = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int32)
    buf = host.to("cuda")
    sink = tsa.stream_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def test_stream_read_rejects_a_ragged_size():
    buf = torch.zeros(17, dtype=torch.uint8, device="cuda")
    with pytest.raises(tsa.TsaError):
        tsa.stream_read(buf)
