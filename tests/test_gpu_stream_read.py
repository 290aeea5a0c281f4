"""The stream-read kernels (a measurement aid, both modes): each must read every 16-byte word once.

The kernel XORs the 32-bit words each lane reads and stores the result only when it equals one
fixed value, so a buffer of zeros with that value in a single word makes the lane that read the
word store it: the sink holds the value exactly when that word was read.
"""
import pytest
import torch

from mla_latent_kv_compress_amd import api

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n16", [1, 7, 1024 * 256, 4 * 1024 * 256 + 5, 3_000_001])
def test_every_word_is_read(n16, mode):
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    magic = MAGIC - (1 << 32)                       # the same bits as a signed int32
    for w in sorted({0, 3, n16 * 4 - 1, (n16 // 2) * 4 + 2, max(0, n16 * 4 - 13)}):
        buf.zero_()
        buf[w] = magic
        sink.zero_()
        api.stream_read(buf, sink, mode)
        torch.cuda.synchronize()
        assert int(sink.item()) == magic, (n16, w)
    buf.zero_()
    sink.zero_()
    api.stream_read(buf, sink, mode)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
