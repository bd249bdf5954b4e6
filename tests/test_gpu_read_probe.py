"""csa2_read_probe (the plain-read yardstick for the full scan) reads every
byte it is given: each of its 512 x 256 threads xor-reduces the 16-byte
words it loads, so the xor of the whole sink equals the xor of the buffer's
32-bit words, which numpy computes independently."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
from tests._gpu import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16 * 7, 16 * 512 * 256 * 4 * 3 + 16 * 5])
def test_read_probe_reads_every_word(nbytes):
    require_gpu()
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((512 * 256,), 7, dtype=torch.int32, device="cuda")
    csa2.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
