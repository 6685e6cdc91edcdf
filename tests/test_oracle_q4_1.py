"""Pins for the oracle's q4_1 decode, q4_1 product and MUL_MAT_ID.

q4_1: W = q*d + m with bf16 d and m per block of 32 consecutive k of one
output column ("NPU engine", "Q4NX chunks"; "Zaya 8B Q4NX on the AMD NPU",
"Round 26").  MUL_MAT_ID reads top-k ids through a stride-17 view ("Zaya 8B",
"The bugs that were the work").
"""
import numpy as np
import pytest

import workloads as wl
from conftest import load_golden


def _explicit_blocks(N, nb, g):
    d_bits = wl.f32_to_bf16_bits(g.uniform(0.001, 0.01, (N, nb)).astype(np.float32))
    m_bits = wl.f32_to_bf16_bits(g.uniform(-0.05, 0.0, (N, nb)).astype(np.float32))
    codes = g.integers(0, 16, size=(N, nb, 32)).astype(np.uint8)
    return d_bits, m_bits, codes, wl.q4_1_blocks_from_parts(d_bits, m_bits, codes)


def test_chunk_size_matches_pages(orc):
    """A 32 x 256 tile of 4-bit codes with a bf16 scale and min per 32 values
    is exactly one 5120-byte chunk: 20 bytes per block."""
    gd = load_golden("q4nx_chunk.txt")
    K, N = gd["tile_cols"], gd["tile_rows"]          # 32 output rows x 256 inputs
    W = wl.normal_f32(np.random.default_rng(0), (K, N), 0.02)
    assert wl.encode_q4_1(W).nbytes == gd["chunk_bytes"]
    assert K * N // 2 + (K * N // 32) * 4 == gd["chunk_bytes"]


def test_decode_closed_form(orc):
    """Blocks built from explicit (d, m, codes): the decoded value at (k, n) is
    codes[n, k//32, k%32] * d + m, element by element."""
    g = np.random.default_rng(21)
    N, nb = 5, 3
    d_bits, m_bits, codes, blocks = _explicit_blocks(N, nb, g)
    W = orc.q4_1_decode(blocks, nb * 32, N)
    d = wl.bf16_bits_to_f32(d_bits).astype(np.float64)
    m = wl.bf16_bits_to_f32(m_bits).astype(np.float64)
    for n in range(N):
        for k in range(nb * 32):
            assert W[k, n] == codes[n, k // 32, k % 32] * d[n, k // 32] + m[n, k // 32]


def test_decode_reconstructs_encoded_weights(orc):
    """The encoder rounds to the nearest code, so decode(encode(W)) is within
    half a step (plus bf16 slack) of W; a wrong nibble order or swapped d/m
    would break this by whole steps."""
    W, blocks = wl.q4_weight(256, 48, seed_index=7)
    Wd = orc.q4_1_decode(blocks, 256, 48)
    x = W.T.reshape(48, 8, 32)
    dq = blocks.reshape(48, 8, 20)
    d = wl.bf16_bits_to_f32(dq[..., 0].astype(np.uint16) | (dq[..., 1].astype(np.uint16) << 8))
    err = np.abs(Wd.T.reshape(48, 8, 32) - x)
    span = x.max(-1) - x.min(-1)
    assert (err <= (0.5 * d + span / 15 * 2 ** -7 + 2 * np.abs(x).max(-1) * 2 ** -8)[..., None]).all()


def test_matmul_equals_numpy_on_decoded(orc):
    g = np.random.default_rng(22)
    K, N, M = 96, 37, 5
    _, _, _, blocks = _explicit_blocks(N, K // 32, g)
    X = wl.normal_f32(g, (M, K))
    Y = orc.q4_1_matmul(X, blocks, K, N)
    ref = X.astype(np.float64) @ orc.q4_1_decode(blocks, K, N)
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def test_block_factorisation_identity(orc):
    """Y = sum_b d*(sum_{k in b} q*x) + m*(sum_{k in b} x) equals the direct
    product (fp64, up to summation order)."""
    g = np.random.default_rng(23)
    K, N, M = 160, 11, 4
    d_bits, m_bits, codes, blocks = _explicit_blocks(N, K // 32, g)
    X = wl.normal_f32(g, (M, K)).astype(np.float64)
    d = wl.bf16_bits_to_f32(d_bits).astype(np.float64)
    mn = wl.bf16_bits_to_f32(m_bits).astype(np.float64)
    Xb = X.reshape(M, K // 32, 32)
    qx = np.einsum("mbj,nbj->mnb", Xb, codes.astype(np.float64))
    ref = (qx * d[None]).sum(-1) + (Xb.sum(-1)[:, None, :] * mn[None]).sum(-1)
    Y = orc.q4_1_matmul(X.astype(np.float32), blocks, K, N)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_zero_scale_blocks_give_min_times_sum(orc):
    g = np.random.default_rng(24)
    N, nb = 3, 2
    d_bits = np.zeros((N, nb), dtype=np.uint16)
    m_bits = wl.f32_to_bf16_bits(g.uniform(-1, 1, (N, nb)).astype(np.float32))
    codes = g.integers(0, 16, size=(N, nb, 32)).astype(np.uint8)
    blocks = wl.q4_1_blocks_from_parts(d_bits, m_bits, codes)
    X = wl.normal_f32(g, (2, 64))
    Y = orc.q4_1_matmul(X, blocks, 64, N)
    mn = wl.bf16_bits_to_f32(m_bits).astype(np.float64)
    xs = X.astype(np.float64).reshape(2, 2, 32).sum(-1)
    assert np.allclose(Y, xs @ mn.T, rtol=1e-13, atol=1e-13)


def test_brute_force_single_block(orc):
    """K = 32, N = 1, pure-Python loop over the block bytes."""
    g = np.random.default_rng(25)
    d_bits, m_bits, codes, blocks = _explicit_blocks(1, 1, g)
    X = wl.normal_f32(g, (3, 32))
    raw = blocks.reshape(20)
    d = float(wl.bf16_bits_to_f32(np.uint16(int(raw[0]) | (int(raw[1]) << 8))))
    mn = float(wl.bf16_bits_to_f32(np.uint16(int(raw[2]) | (int(raw[3]) << 8))))
    Y = orc.q4_1_matmul(X, blocks, 32, 1)
    for r in range(3):
        s = 0.0
        for j in range(32):
            byte = int(raw[4 + (j % 16)])
            q = (byte & 15) if j < 16 else (byte >> 4)
            s += float(X[r, j]) * (q * d + mn)
        assert abs(Y[r, 0] - s) <= 1e-12 * max(1.0, abs(s))


def test_sampled_matches_full(orc):
    W, blocks = wl.q4_weight(128, 40, seed_index=3)
    X = wl.q4_activations(6, 128)
    Y = orc.q4_1_matmul(X, blocks, 128, 40)
    im = np.array([0, 5, 2])
    in_ = np.array([39, 0, 17])
    assert np.array_equal(orc.q4_1_matmul_at(X, blocks, 128, 40, im, in_), Y[im, in_])


def test_fp32_sequential_error_is_visible(orc):
    """Diagnostic: a naive fp32 sequential sum at K = 14336 differs from the
    fp64 oracle by far more than fp64 rounding, so the fp64 reference is the
    one a 1e-5 Frobenius gate needs (not a parity gate itself)."""
    g = np.random.default_rng(26)
    K = 14336
    W, blocks = wl.q4_weight(K, 4, seed_index=9)
    X = wl.normal_f32(g, (1, K))
    Y = orc.q4_1_matmul(X, blocks, K, 4)
    Wd = orc.q4_1_decode(blocks, K, 4).astype(np.float32)
    acc = np.zeros(4, dtype=np.float32)
    for k in range(K):
        acc = (acc + X[0, k] * Wd[k]).astype(np.float32)
    rel = np.linalg.norm(acc - Y[0]) / np.linalg.norm(Y[0])
    assert 1e-9 < rel < 1e-4


# ------------------------------------------------------------ MUL_MAT_ID ---

def _small_moe(g, E=6, K=64, N=24, T=10, stride=17, n_used=3):
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(max(E, stride))[:stride] % E for _ in range(T)]).astype(np.int32)
    return experts, X, ids


def test_moe_all_same_expert_is_plain_matmul(orc):
    g = np.random.default_rng(31)
    E, K, N, T = 6, 64, 24, 10
    experts, X, ids = _small_moe(g, E, K, N, T)
    ids[:] = 4
    Y = orc.q4_1_matmul_id(X, experts, E, K, N, ids, 3)
    ref = orc.q4_1_matmul(X, experts[4], K, N)
    for s in range(3):
        assert np.array_equal(Y[:, s], ref)


def test_moe_strided_ids_and_tail(orc):
    """Only the first n_used ids of each stride-17 row matter: a contiguous
    copy of those columns gives the same result, rewriting the tail changes
    nothing, and reading the buffer contiguously (the pages' bug) differs."""
    gd = load_golden("moe_ids_stride.txt")
    stride = gd["experts_per_row"]
    assert stride * 4 == gd["row_stride_bytes"]
    g = np.random.default_rng(32)
    E, K, N, T, n_used = 20, 64, 16, 12, 4
    experts, X, ids = _small_moe(g, E, K, N, T, stride, n_used)
    Y = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
    Yc = orc.q4_1_matmul_id(X, experts, E, K, N, np.ascontiguousarray(ids[:, :n_used]), n_used)
    assert np.array_equal(Y, Yc)
    ids2 = ids.copy()
    ids2[:, n_used:] = (ids2[:, n_used:] + 7) % E
    assert np.array_equal(Y, orc.q4_1_matmul_id(X, experts, E, K, N, ids2, n_used))
    wrong = np.ascontiguousarray(ids.reshape(-1)[: T * n_used].reshape(T, n_used))
    assert not np.array_equal(Y, orc.q4_1_matmul_id(X, experts, E, K, N, wrong, n_used))
    for t in range(T):
        for s in range(n_used):
            assert np.array_equal(Y[t, s], orc.q4_1_matmul(X[t:t + 1], experts[ids[t, s]], K, N)[0])


def test_moe_token_permutation_and_single_slot(orc):
    g = np.random.default_rng(33)
    E, K, N, T = 9, 32, 16, 8
    experts, X, ids = _small_moe(g, E, K, N, T)
    perm = g.permutation(T)
    Y = orc.q4_1_matmul_id(X, experts, E, K, N, ids, 2)
    Yp = orc.q4_1_matmul_id(X[perm], experts, E, K, N, ids[perm], 2)
    assert np.array_equal(Yp, Y[perm])
    Y1 = orc.q4_1_matmul_id(X, experts, E, K, N, ids, 1)
    assert np.array_equal(Y1[:, 0], Y[:, 0])


def test_moe_rejects_bad_id(orc):
    g = np.random.default_rng(34)
    experts, X, ids = _small_moe(g, 6, 32, 16, 4)
    ids[2, 1] = 6
    with pytest.raises(ValueError):
        orc.q4_1_matmul_id(X, experts, 6, 32, 16, ids, 3)


def test_moe_sampled(orc):
    g = np.random.default_rng(35)
    E, K, N, T = 7, 64, 16, 9
    experts, X, ids = _small_moe(g, E, K, N, T)
    Y = orc.q4_1_matmul_id(X, experts, E, K, N, ids, 3)
    it = np.array([0, 8, 4])
    is_ = np.array([2, 0, 1])
    in_ = np.array([15, 3, 0])
    got = orc.q4_1_matmul_id_at(X, experts, E, K, N, ids, it, is_, in_)
    assert np.array_equal(got, Y[it, is_, in_])


# ------------------------------------- MUL_MAT_ID, per-slot activations ---
# Down experts read an activation row of their own per (token, slot), the
# per-expert form [k, n_expert_used, ntokens] ("Zaya 8B Q4NX on the AMD NPU",
# "What's next": reading token t's shared row for every slot was the bug).

def test_moe_per_slot_reduces_to_shared(orc):
    """Every slot row equal to the token's row: the shared form's result."""
    g = np.random.default_rng(41)
    E, K, N, T, n_used = 7, 64, 24, 9, 3
    experts, X, ids = _small_moe(g, E, K, N, T, n_used=n_used)
    X3 = np.repeat(X[:, None, :], n_used, axis=1)
    assert np.array_equal(orc.q4_1_matmul_id(X3, experts, E, K, N, ids, n_used),
                          orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used))


def test_moe_per_slot_against_numpy(orc):
    """Each (t, s) output is numpy's fp64 product of that slot's row with the
    decoded expert (decode pinned by its closed form); reading slot 0's row for
    every slot (the pages' bug) gives a different result."""
    g = np.random.default_rng(42)
    E, K, N, T, n_used = 6, 96, 20, 7, 4
    experts, _, ids = _small_moe(g, E, K, N, T, n_used=n_used)
    X3 = wl.normal_f32(g, (T, n_used, K))
    Y = orc.q4_1_matmul_id(X3, experts, E, K, N, ids, n_used)
    W = [orc.q4_1_decode(experts[e], K, N) for e in range(E)]
    for t in range(T):
        for s in range(n_used):
            ref = X3[t, s].astype(np.float64) @ W[ids[t, s]]
            assert np.allclose(Y[t, s], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    bug = orc.q4_1_matmul_id(np.ascontiguousarray(X3[:, 0]), experts, E, K, N, ids, n_used)
    assert np.array_equal(bug[:, 0], Y[:, 0])
    assert not np.allclose(bug[:, 1:], Y[:, 1:])


def test_moe_per_slot_permutation_and_sampled(orc):
    """Permuting the slots (ids and rows together) permutes the outputs; the
    sampled form reads the same rows."""
    g = np.random.default_rng(43)
    E, K, N, T, n_used = 8, 64, 16, 6, 5
    experts, _, ids = _small_moe(g, E, K, N, T, n_used=n_used)
    X3 = wl.normal_f32(g, (T, n_used, K))
    Y = orc.q4_1_matmul_id(X3, experts, E, K, N, ids, n_used)
    perm = g.permutation(n_used)
    ids_p = ids.copy()
    ids_p[:, :n_used] = ids[:, perm]
    Yp = orc.q4_1_matmul_id(np.ascontiguousarray(X3[:, perm]), experts, E, K, N, ids_p, n_used)
    assert np.array_equal(Yp, Y[:, perm])
    it = np.array([0, 5, 3, 2])
    is_ = np.array([4, 0, 2, 1])
    in_ = np.array([15, 3, 0, 7])
    got = orc.q4_1_matmul_id_at(X3, experts, E, K, N, ids, it, is_, in_, n_used=n_used)
    assert np.array_equal(got, Y[it, is_, in_])


# ------------------------- q4_1 weights x per-row int8 activations ---

def test_q4_q8_against_numpy(orc):
    """Y = diag(sa) (Xq @ W) with W decoded by its closed form (pinned above):
    numpy fp64 on the decoded weight, including codes 0/15, d = 0 blocks and
    activation codes +-127."""
    g = np.random.default_rng(71)
    M, K, N = 5, 160, 19
    W = wl.normal_f32(g, (K, N), 0.02)
    blocks = wl.encode_q4_1(W)
    blocks[3, 1, :2] = 0                         # d = 0 block
    Xq = g.integers(-127, 128, (M, K)).astype(np.int8)
    Xq[0, :7] = 127
    Xq[1, 40:50] = -127
    sa = g.uniform(0.001, 0.05, M).astype(np.float32)
    Y = orc.q4_1_matmul_q8(Xq, sa, blocks, K, N)
    ref = (Xq.astype(np.float64) @ orc.q4_1_decode(blocks, K, N)) * sa.astype(np.float64)[:, None]
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_q4_q8_integer_block_form(orc):
    """The block form with Python integers for the dots and row sums on one
    block per column, from explicit (d, m, codes): exact to fp64 rounding."""
    g = np.random.default_rng(72)
    N, nb = 3, 2
    d_bits, m_bits, codes, blocks = _explicit_blocks(N, nb, g)
    K = 32 * nb
    Xq = g.integers(-127, 128, (2, K)).astype(np.int8)
    sa = np.array([0.5, 0.25], dtype=np.float32)
    Y = orc.q4_1_matmul_q8(Xq, sa, blocks, K, N)
    for m in range(2):
        for n in range(N):
            tot = 0.0
            for b in range(nb):
                xs = [int(v) for v in Xq[m, 32 * b:32 * b + 32]]
                D = sum(int(c) * x for c, x in zip(codes[n, b], xs))
                S = sum(xs)
                tot += float(wl.bf16_bits_to_f32(d_bits[n, b])) * D + float(wl.bf16_bits_to_f32(m_bits[n, b])) * S
            assert Y[m, n] == pytest.approx(float(sa[m]) * tot, rel=1e-15, abs=1e-300)


def test_q4_q8_matches_fp32_activation_path(orc):
    """With activations that are exactly their int8 codes times the row scale,
    the fp32-activation product (pinned above) gives the same result."""
    g = np.random.default_rng(73)
    M, K, N = 3, 96, 11
    blocks = wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02))
    Xq = g.integers(-127, 128, (M, K)).astype(np.int8)
    sa = np.array([1.0, 0.5, 2.0 ** -7], dtype=np.float32)
    X = (Xq.astype(np.float32) * sa[:, None]).astype(np.float32)     # exact: power-of-two scales
    assert np.allclose(orc.q4_1_matmul_q8(Xq, sa, blocks, K, N), orc.q4_1_matmul(X, blocks, K, N),
                       rtol=1e-12, atol=1e-15)
