"""The streaming-read probe the bandwidth floors are measured with: every
16-byte chunk is read exactly once (each workgroup's XOR of its chunks
matches the host's), including a ragged last pass of the grid-stride loop."""
import numpy as np
import pytest

from gpu_util import to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (4096 * 16 + 48, 7), (2301952, 1024)])
def test_read_probe_reads_every_chunk_once(nbytes, wg):
    import torch
    import int8_bit_weight_amd as q
    g = np.random.default_rng(nbytes + wg)
    host = g.integers(0, 256, nbytes, dtype=np.int64).astype(np.uint8)
    sink = torch.full((wg,), 7, dtype=torch.int32, device=torch_dev())
    q.read_probe(to_dev(host), sink, wg)
    c = host.view(np.int32).reshape(-1, 4)
    c = c[:, 0] ^ c[:, 1] ^ c[:, 2] ^ c[:, 3]
    w = (np.arange(c.size) % (wg * 256)) // 256
    want = np.zeros(wg, dtype=np.int32)
    for i in range(wg):
        want[i] = np.bitwise_xor.reduce(c[w == i]) if (w == i).any() else 0
    assert np.array_equal(to_np(sink), want)
