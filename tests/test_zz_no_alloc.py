"""The allocation-free MUL_MAT_ID entry point (q4_1_matmul_id_noalloc),
through the C ABI: the same bits as q4_1_matmul_id with a caller workspace,
on two calls in a row (the second smaller, so stale contents of the shared
scratch array would show), and within the 1e-5 gate of the fp64 oracle."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu


def _case(E, K, N, T, n_used, seed):
    g = np.random.default_rng(seed)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(max(E, 17))[:17] % E for _ in range(T)]).astype(np.int32)
    return experts, X, ids


def test_noalloc_matches_workspace_call_twice(orc):
    import int8_bit_weight_amd as q
    for E, K, N, T, n_used, seed in [(16, 256, 300, 100, 4, 1), (5, 96, 40, 7, 3, 2)]:
        experts, X, ids = _case(E, K, N, T, n_used, seed)
        buf, st = q.q4_1_repack_experts(to_dev(experts), K, N)
        Xd, idd = to_dev(X), to_dev(ids)
        a = to_np(q.q4_1_matmul_id_noalloc(Xd, buf, E, K, N, st, idd, n_used))
        assert q.last_variant() == "q4_moe_m32"
        b = to_np(q.q4_1_matmul_id(Xd, buf, E, K, N, st, idd, n_used))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (E, K, N, T)
        ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
        assert np.linalg.norm(a.astype(np.float64) - ref) <= 1e-5 * np.linalg.norm(ref)
