"""GPU parity of an lm_head-shaped projection (K = 1024 onto N = 151936
columns, the Qwen3-0.6B vocabulary) through the C ABI.

One large streaming matmul per decoded token: the int8 path (packB of fp32
N(0, 0.02) weights, per-row quantisation inside the product, fp32 output) at
M = 1 and 16, and the q4_1 path at M = 1 and 16.  The full 151936-column
output is produced in one call; the oracle evaluates sampled columns (every
column is independent: packB and q4_1 blocks are per column), plus the first
and last columns and the last 16-column strip, which is ragged (151936 is a
multiple of 16 but not of the kernels' wider column groups).

Bars: packed codes, scales and column sums at the sampled columns, the
quantised rows and the int32 product bit-exact; fp32 output max|dY| <= 2e-6 *
max|Y|; q4_1 relative Frobenius error <= 1e-5 on the sampled columns.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import frob_rel_err, max_rel_err, to_dev, to_np, torch_dev, unpack_int8_codes

pytestmark = pytest.mark.gpu

F32_TOL = 2e-6
Q4_TOL = 1e-5


@pytest.fixture(scope="module")
def q():
    import int8_bit_weight_amd as q
    return q


@pytest.fixture(scope="module")
def weight():
    return wl.lm_head_weight()


def _columns(N, n=512, seed=0):
    g = np.random.default_rng(seed)
    cols = np.concatenate([g.choice(N, n, replace=False), [0, 1], N - 16 + np.arange(16)])
    return np.unique(cols.astype(np.int64))


def test_lm_head_int8(q, orc, weight):
    import torch
    K, N = weight.shape
    dev = torch_dev()
    p = q.pack_b_int8(to_dev(weight))
    cols = _columns(N, seed=1)
    Wc = np.ascontiguousarray(weight[:, cols])
    Qb, sb, cb = orc.pack_b_int8(Wc)
    codes, scale, colsum, _ = unpack_int8_codes(to_np(p.data), K, N)
    assert np.array_equal(codes[:K, cols], Qb)
    assert np.array_equal(scale[cols].view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(colsum[cols], cb)
    del codes
    for M in wl.LM_HEAD_ROWS:
        X = wl.lm_head_activations(M, seed_index=M)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        y32 = torch.empty((M, N), dtype=torch.int32, device=dev)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        rs = torch.empty((M,), dtype=torch.float32, device=dev)
        q.int8_gemm_dynamic(to_dev(X), p, out_f32=y, out_i32=y32, xq_out=xq, rs_out=rs)
        assert q.last_variant() == "int8_dynamic_wide_m16p", q.last_variant()
        Qa, sa = orc.quantize_rows_int8(X)
        assert np.array_equal(to_np(xq), Qa)
        assert np.array_equal(to_np(rs).view(np.uint32), sa.view(np.uint32))
        Y64 = orc.int8_gemm_i64(Qa, 0, Qb, 0)
        assert np.array_equal(to_np(y32)[:, cols], Y64.astype(np.int32)), M
        ref = orc.epilogue_f64(Y64, sa, sb)
        got = to_np(y)
        assert np.isfinite(got).all()
        assert max_rel_err(got[:, cols], ref) <= F32_TOL, M


def test_lm_head_q4_1(q, orc, weight):
    import torch
    K, N = weight.shape
    dev = torch_dev()
    blocks = wl.encode_q4_1(weight)                       # [N, K/32, 20]
    p = q.q4_1_repack(to_dev(blocks.reshape(-1)), K, N)
    cols = _columns(N, seed=2)
    bc = np.ascontiguousarray(blocks[cols])
    for M in wl.LM_HEAD_ROWS:
        X = wl.lm_head_activations(M, seed_index=100 + M)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = q.workspace(q.lib.qmm_q4_1_matmul_workspace_bytes(M, K, N), dev)
        q.q4_1_matmul(to_dev(X), p, out=y, ws=ws)
        assert q.last_variant() == ("q4_gemv_m1_wide" if M == 1 else "q4_mm16_wide"), q.last_variant()
        got = to_np(y)
        assert np.isfinite(got).all()
        ref = orc.q4_1_matmul(X, bc, K, len(cols))
        assert frob_rel_err(got[:, cols], ref) <= Q4_TOL, M
