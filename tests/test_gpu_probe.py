"""The streaming-read probe the bandwidth floors are measured with: every
16-byte chunk is read exactly once (each workgroup's XOR of its chunks
matches the host's), for 1 to 8 loads in flight per lane, including ragged
last blocks and workgroups without a block."""
import numpy as np
import pytest

from gpu_util import to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (4096 * 16 + 48, 7), (2301952, 1024), (131072, 300)])
@pytest.mark.parametrize("u", [1, 2, 4, 8])
def test_read_probe_reads_every_chunk_once(nbytes, wg, u):
    import torch
    from int8_bit_weight_amd.probe import read_probe
    g = np.random.default_rng(nbytes + wg + u)
    host = g.integers(0, 256, nbytes, dtype=np.int64).astype(np.uint8)
    sink = torch.full((wg,), 7, dtype=torch.int32, device=torch_dev())
    read_probe(to_dev(host), sink, wg, loads_per_lane=u)
    c = host.view(np.int32).reshape(-1, 4)
    c = c[:, 0] ^ c[:, 1] ^ c[:, 2] ^ c[:, 3]
    w = (np.arange(c.size) // (256 * u)) % wg        # block -> workgroup
    want = np.zeros(wg, dtype=np.int32)
    for i in range(wg):
        want[i] = np.bitwise_xor.reduce(c[w == i]) if (w == i).any() else 0
    assert np.array_equal(to_np(sink), want)
