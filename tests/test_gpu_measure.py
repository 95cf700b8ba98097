"""The measurement kernel behind the bench's HBM ceiling (ql_stream_read):
one pass reads every 16-byte word of the buffer exactly once, so the XOR of
its per-thread results equals the XOR of all 32-bit words of the buffer,
computed on the host.  Sizes below, at and past the grid's width, not
multiples of it, and a buffer at a 16-byte offset into an allocation."""

import numpy as np
import pytest
import torch

from quantized_base_lora_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [1, 7, 65535, 65536, 65537, 3 * 65536 + 5, 1 << 20])
@pytest.mark.parametrize("offset_words", [0, 1])
def test_stream_read_visits_every_word(lib, words, offset_words):
    g = np.random.default_rng(words + offset_words)
    host = g.integers(0, 2 ** 32, size=4 * (words + offset_words), dtype=np.uint64).astype(np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    buf = dev[4 * offset_words:]
    sink = torch.full((B.STREAM_READ_THREADS,), -1, dtype=torch.int32, device="cuda")
    B.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = int(np.bitwise_xor.reduce(host[4 * offset_words:]))
    assert got == want, (words, offset_words, hex(got), hex(want))
