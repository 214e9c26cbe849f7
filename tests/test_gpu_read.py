"""The streaming-read reference kernel reads every byte once: the XOR of all
32-bit words it folds into the sink equals the host's, for sizes with and
without a partial 16-byte tail and spanning many grid-stride passes."""
import numpy as np
import pytest

from helpers import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [1, 3, 4, 5, 1023, 4096 * 1024 + 7, 7_000_003])
def test_read_bandwidth_reads_every_word_once(trellis_lib, words):
    import torch
    announce(f"read_bandwidth over {words} words")
    g = np.random.default_rng(words)
    host = g.integers(0, 1 << 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    trellis_lib.read_bandwidth(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == int(want)
