"""The plain-read yardstick (medusa_stream_read) reads every 16 bytes of its
buffer: one nonzero word planted in a zero buffer is seen (the thread that
read it writes its fold to the sink) wherever it lies, including the tail
past the last full round of the four-loads-per-thread loop."""

import pytest
import torch

from speculative_decoding_heads_amd import medusa as M
from tests.helpers import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("nbytes", [16, 4096, 512 * 256 * 16 * 4 + 48, 134217728])
def test_every_word_is_read(nbytes):
    say("stream_read", nbytes)
    n = nbytes // 4
    buf = torch.zeros(n, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for pos in sorted({0, n // 3, n - 5, n - 1}):
        buf.zero_()
        buf[pos] = 0x5A5A1234
        sink.fill_(7)
        M.medusa_stream_read(buf, sink, never=0x5A5A1234)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0x5A5A1234, pos
        # a value no fold takes: nothing written
        sink.fill_(7)
        M.medusa_stream_read(buf, sink, never=0x0F0F0F0F)
        torch.cuda.synchronize()
        assert int(sink.item()) == 7, pos
