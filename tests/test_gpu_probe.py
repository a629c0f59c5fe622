"""pg_read_probe, the streaming-read measurement utility: every 16-byte word
of the buffer is read exactly once (the XOR of the per-block sink words equals
the XOR of all 32-bit words of the buffer), for a ragged size and for a
buffer smaller than the grid."""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4 * (3 * 1024 * 1024 // 16 + 3), 4 * 1000])
def test_read_probe_reads_every_word_once(n_words):
    rng = np.random.default_rng(7)
    host = rng.integers(0, 2**32, size=n_words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    pg.pg_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    assert got == want
