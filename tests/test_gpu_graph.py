"""HIP graph capture of the entry points, as the benchmark times them.

One graph holds a call of each kind of launch: the fused int8 decode over a
few strips, the persistent wide int8 decode (with the rows quantised inside),
the q4_1 k-split product and its split sum, the persistent q4_1 16-row
product, and MUL_MAT_ID (the routing launch, then the grouped product).  The
graph is replayed three times, with eager work that overwrites every output
between the replays, and each replay must give the eager call's outputs bit
for bit (every kernel here is deterministic).
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import int8_bit_weight_amd as q
    return q


def test_graph_replays_match_eager(q):
    import torch
    dev = torch_dev()
    g = np.random.default_rng(2024)
    calls, outs = [], []

    # int8_gemm_dynamic: fused decode (192 strips) and the persistent wide form (4100 strips)
    for M, K, N in ((32, 1024, 3072), (16, 1024, 16 * 4100)):
        pk = q.pack_b_int8(to_dev(wl.normal_f32(g, (K, N), 0.02)))
        X = to_dev(wl.normal_f32(g, (M, K)))
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        calls.append(lambda X=X, pk=pk, Y=Y: q.int8_gemm_dynamic(X, pk, out_f32=Y))
        outs.append(Y)

    # q4_1_matmul: four k splits and the split sum; the persistent 16-row form
    for M, K, N in ((16, 4096, 1024), (16, 1024, 16 * 4100)):
        _, blocks = wl.q4_weight(K, N, seed_index=M + K + N)
        pk = q.q4_1_repack(to_dev(blocks.reshape(-1)), K, N)
        X = to_dev(wl.q4_activations(M, K, seed_index=M + K))
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
        calls.append(lambda X=X, pk=pk, Y=Y, ws=ws: q.q4_1_matmul(X, pk, out=Y, ws=ws))
        outs.append(Y)

    # MUL_MAT_ID: 16 experts, 64 tokens, top-4 of rows of stride 17
    E, K, N, T, n_used = 16, 256, 128, 64, 4
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    ids = to_dev(np.stack([g.permutation(17) % E for _ in range(T)]).astype(np.int32))
    X = to_dev(wl.normal_f32(g, (T, K)))
    Y = torch.empty((T, n_used, N), dtype=torch.float32, device=dev)
    ws = q.workspace(q.lib.qmm_q4_1_matmul_id_workspace_bytes(T, n_used, E, K, N), dev)
    calls.append(lambda: q.q4_1_matmul_id(X, buf, E, K, N, estride, ids, n_used, out=Y, ws=ws))
    outs.append(Y)

    def run():
        for c in calls:
            c()

    run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in outs]
    assert all(torch.isfinite(r).all() for r in ref)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, r) in enumerate(zip(outs, ref)):
            assert torch.equal(y, r), (rep, i)
