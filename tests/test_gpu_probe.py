"""The plain streaming read (the measurement ceiling of the matmuls) reads
every byte it is given exactly once: the xor of the words its blocks write
equals the xor of the buffer's 32-bit words, on sizes that are a whole
number of chunks, a ragged tail, and less than one chunk."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 8192 * 4 * 512, 5320704, 28350464 + 48])
def test_read_probe_reads_every_word_once(q4, nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    q4.read_probe(src, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
