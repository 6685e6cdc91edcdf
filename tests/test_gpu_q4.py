"""GPU parity of the q4_1 path (repack, product, MUL_MAT_ID) against the CPU
oracle, through the C ABI.

The repack is a byte permutation and must be exact.  Products must satisfy
||Y - Y_ref||_F <= 1e-5 * ||Y_ref||_F against the oracle's fp64 result on the
same codes.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import canonical_q4_parts, to_dev, to_np, torch_dev, unpack_q4_records

pytestmark = pytest.mark.gpu

FROB_TOL = 1e-5


def _abs_scale(orc, X, blocks, K, N):
    """|X| @ |W|: the magnitude of the terms each output sums."""
    return np.abs(X.astype(np.float64)) @ np.abs(orc.q4_1_decode(blocks, K, N))


def _check(got, ref):
    """The 1e-5 relative Frobenius gate against ||Y_ref||_F."""
    err = np.linalg.norm(got.astype(np.float64) - ref)
    denom = np.linalg.norm(ref)
    assert err <= FROB_TOL * denom, (err / max(denom, 1e-300))


def _check_edge(got, ref, scale, K, N):
    """The same 1e-5 gate for the two literal edge shapes only: one 32-k block
    (K = 32) or one output column (N = 1).  There d*sum(q*x) and m*sum(x) of
    a single block can cancel to an output far smaller than the two terms,
    and fp32 rounding of the terms is then large relative to that output
    though tiny relative to the terms, so the gate is taken relative to
    max(||Y_ref||_F, ||(|X| @ |W|)||_F)."""
    assert K == 32 or N == 1, "the term-size gate is for one-block or one-column shapes only"
    err = np.linalg.norm(got.astype(np.float64) - ref)
    denom = max(np.linalg.norm(ref), np.linalg.norm(scale))
    assert err <= FROB_TOL * denom, (err / max(denom, 1e-300))


def _gate(got, ref, scale, K, N):
    """Strict gate, or the edge-shape gate for K = 32 or N = 1."""
    if K == 32 or N == 1:
        _check_edge(got, ref, scale, K, N)
    else:
        _check(got, ref)


@pytest.fixture(scope="module")
def q():
    import int8_bit_weight_amd as q
    return q


def _blocks(K, N, seed, zero_cols=(), zero_scale_blocks=False):
    W, blocks = wl.q4_weight(K, N, seed_index=seed)
    blocks = blocks.copy()
    for c in zero_cols:
        if c < N:
            blocks[c] = 0                      # d = m = 0, codes 0: an all-zero column
    if zero_scale_blocks and N > 1 and K >= 64:
        blocks[1, 1, 0:2] = 0                  # d = 0 on one block: value m everywhere
    return blocks


def _repack(q, blocks, K, N):
    return q.q4_1_repack(to_dev(blocks.reshape(-1)), K, N)


@pytest.mark.parametrize("K,N", [(4096, 64), (96, 17), (32, 1), (160, 300)])
def test_repack_is_exact_permutation(q, K, N):
    blocks = _blocks(K, N, seed=K + N)
    p = _repack(q, blocks, K, N)
    assert q.last_variant() == "q4_repack"
    codes, d, m = unpack_q4_records(to_np(p.data), K, N)
    rc, rd, rm = canonical_q4_parts(blocks, K, N)
    assert np.array_equal(codes, rc)
    assert np.array_equal(d, rd) and np.array_equal(m, rm)
    raw = to_np(p.data)
    NB, NS = K // 32, (N + 15) // 16
    NQ = (NB + 3) // 4
    assert raw.size == 64 + NS * NQ * 1280 == q.lib.qmm_q4_1_packed_bytes(K, N)


def _matmul_case(q, orc, M, K, N, seed, variant=None, **kw):
    blocks = _blocks(K, N, seed, **kw)
    X = wl.q4_activations(M, K, seed_index=seed)
    p = _repack(q, blocks, K, N)
    Y = q.q4_1_matmul(to_dev(X), p)
    if variant is not None:
        assert q.last_variant() == variant
    got = to_np(Y)
    ref = orc.q4_1_matmul(X, blocks, K, N)
    if K == 32 or N == 1:
        _check_edge(got, ref, _abs_scale(orc, X, blocks, K, N), K, N)
    else:
        _check(got, ref)
    return got, ref


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (1, 96, 17), (2, 64, 15), (16, 4096, 64), (17, 160, 300),
                                   (33, 256, 40), (5, 1024, 33), (16, 32 * 44, 272), (64, 128, 48),
                                   (20, 2048, 303)])
def test_q4_matmul_small(q, orc, M, K, N):
    _matmul_case(q, orc, M, K, N, seed=M * 7 + K + N, zero_cols=(3,), zero_scale_blocks=True)


@pytest.mark.parametrize("M,variant", [(33, "q4_gemv_m1"), (49, "q4_mm_m32"), (65, "q4_gemv_m1"),
                                       (36, "q4_gemv_m4"), (44, "q4_mm16")])
def test_q4_matmul_row_remainders(q, orc, M, variant):
    """Regression: rows run 32 per launch and the last launch is planned for
    its own row count (1 row: the one-row kernel; 4: the M <= 4 kernel; 12:
    the 5..16 kernel; 17: two 16-row tiles), so the 17..32-row kernel never
    multiplies a row tile without rows.  Ragged N, several k splits."""
    _matmul_case(q, orc, M, 1024, 300, seed=M, variant=variant, zero_cols=(3,), zero_scale_blocks=True)


@pytest.mark.parametrize("K,N", [(1024, 16400), (512, 16389), (96, 16390), (1024, 16384)])
def test_q4_matmul_one_row_wide(q, orc, K, N):
    """M = 1 over >= 1024 strips with at most 8 records each (an lm_head's
    shape class): a wavefront per strip over its whole k range, 8 strips per
    workgroup.  Ragged N (a last workgroup of fewer strips), 4 and 1 records
    per strip, zero columns and zero-scale blocks, aligned and unaligned
    activations, at the 1e-5 bound."""
    import torch
    seed = K + N
    got, ref = _matmul_case(q, orc, 1, K, N, seed=seed, variant="q4_gemv_m1_wide", zero_cols=(3,),
                            zero_scale_blocks=True)
    blocks = _blocks(K, N, seed, zero_cols=(3,), zero_scale_blocks=True)
    p = _repack(q, blocks, K, N)
    X = wl.q4_activations(1, K, seed_index=seed)
    Xw = torch.zeros((1, K + 1), dtype=torch.float32, device=torch_dev())
    Xw[:, 1:] = to_dev(X)
    c = to_np(q.q4_1_matmul(Xw[:, 1:], p))
    assert q.last_variant() == "q4_gemv_m1_wide"
    assert np.array_equal(c.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(16, 96, 131200), (5, 512, 65557), (12, 160, 70001), (16, 1024, 65600)])
def test_q4_matmul_rows_wide(q, orc, M, K, N):
    """5 <= M <= 16 over more than 4096 strips with at most 8 records each
    (an lm_head's shape class): the persistent form, one workgroup per CU
    over a contiguous run of strips, each wavefront running its strips in
    turn with the next strip's records loading.  1, 4, 2 and 8 records per
    strip (160 = 5 blocks: a ragged last record), ragged N (a last
    wavefront with fewer strips), zero columns and zero-scale blocks, at the
    1e-5 bound; unaligned activations and a second call give the same
    bits."""
    import torch
    seed = M + K + N
    got, ref = _matmul_case(q, orc, M, K, N, seed=seed, variant="q4_mm16_wide", zero_cols=(3, N - 1),
                            zero_scale_blocks=True)
    blocks = _blocks(K, N, seed, zero_cols=(3, N - 1), zero_scale_blocks=True)
    p = _repack(q, blocks, K, N)
    X = wl.q4_activations(M, K, seed_index=seed)
    again = to_np(q.q4_1_matmul(to_dev(X), p))
    assert np.array_equal(again.view(np.uint32), got.view(np.uint32))
    Xw = torch.zeros((M, K + 1), dtype=torch.float32, device=torch_dev())
    Xw[:, 1:] = to_dev(X)
    c = to_np(q.q4_1_matmul(Xw[:, 1:], p))
    assert q.last_variant() == "q4_mm16_wide"
    assert np.array_equal(c.view(np.uint32), got.view(np.uint32))


def test_q4_matmul_rows_wide_threshold(q, orc):
    """4096 strips still take the k-split kernel (one workgroup per CU);
    4097 take the persistent form.  Both at the 1e-5 bound."""
    _matmul_case(q, orc, 16, 128, 16 * 4096, seed=5, variant="q4_mm16")
    _matmul_case(q, orc, 16, 128, 16 * 4096 + 1, seed=6, variant="q4_mm16_wide")


def test_q4_matmul_one_row_paths(q, orc):
    """M = 1: the one-launch kernel (aligned and unaligned activations, bitwise
    repeatable), its fallback when a wavefront would hold more than 8 records,
    and M = 4 at a ragged shape."""
    import torch
    K, N = 4096, 96
    blocks = _blocks(K, N, seed=11)
    p = _repack(q, blocks, K, N)
    X = wl.q4_activations(1, K, seed_index=11)
    ref = orc.q4_1_matmul(X, blocks, K, N)
    a = to_np(q.q4_1_matmul(to_dev(X), p))
    assert q.last_variant() == "q4_gemv_m1"
    _check(a, ref)
    b = to_np(q.q4_1_matmul(to_dev(X), p))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # activations one float past a 16-byte boundary: scalar loads
    Xw = torch.zeros((1, K + 1), dtype=torch.float32, device=torch_dev())
    Xw[:, 1:] = to_dev(X)
    c = to_np(q.q4_1_matmul(Xw[:, 1:], p))
    assert q.last_variant() == "q4_gemv_m1"
    _check(c, ref)
    # 160 records over 16 wavefronts: more than 8 each
    K2, N2 = 20480, 40
    blocks2 = _blocks(K2, N2, seed=12)
    p2 = _repack(q, blocks2, K2, N2)
    X2 = wl.q4_activations(1, K2, seed_index=12)
    got2 = to_np(q.q4_1_matmul(to_dev(X2), p2))
    assert q.last_variant() == "q4_gemv_m4"
    _check(got2, orc.q4_1_matmul(X2, blocks2, K2, N2))
    # four rows, K not a multiple of 128, N not a multiple of 16
    K3, N3 = 160, 33
    blocks3 = _blocks(K3, N3, seed=13, zero_cols=(3,), zero_scale_blocks=True)
    p3 = _repack(q, blocks3, K3, N3)
    X3 = wl.q4_activations(4, K3, seed_index=13)
    got3 = to_np(q.q4_1_matmul(to_dev(X3), p3))
    assert q.last_variant() == "q4_gemv_m4"
    _check(got3, orc.q4_1_matmul(X3, blocks3, K3, N3))


@pytest.mark.parametrize("M,K,N,aligned", [(16, 1440, 300, True), (9, 1440, 300, False), (16, 256, 40, False),
                                           (5, 32 * 37, 17, True), (12, 8192, 48, True), (16, 1440, 301, True),
                                           (7, 4096, 18, False)])
def test_q4_matmul_m16_paths(q, orc, M, K, N, aligned):
    """5 <= M <= 16: whole k range staged at once.  K = 1440 (45 blocks):
    two k splits of 6 records, the second with a partial last record and two
    padding records; K = 256: one split, no second kernel; K = 8192: eight
    splits; N not a multiple of the workgroup's 256 columns; activations one
    float past a 16-byte boundary (scalar loads)."""
    import torch
    blocks = _blocks(K, N, seed=M + K + N, zero_cols=(1,), zero_scale_blocks=True)
    p = _repack(q, blocks, K, N)
    X = wl.q4_activations(M, K, seed_index=M + K)
    Xd = to_dev(X)
    if not aligned:
        Xw = torch.zeros((M, K + 1), dtype=torch.float32, device=torch_dev())
        Xw[:, 1:] = Xd
        Xd = Xw[:, 1:]
    got = to_np(q.q4_1_matmul(Xd, p))
    assert q.last_variant() == "q4_mm16"
    _check(got, orc.q4_1_matmul(X, blocks, K, N))


@pytest.mark.parametrize("M,K,N", [(16, 1440, 300), (20, 2048, 300), (16, 4096, 256)])
def test_q4_matmul_strided_output(q, orc, M, K, N):
    """k-split sums written into an output of row stride N + 3 (no 16-byte
    stores) and into one offset by a float: the same bits as the contiguous
    output, and the columns past N untouched."""
    import torch
    dev = torch_dev()
    blocks = _blocks(K, N, seed=M + K + N)
    p = _repack(q, blocks, K, N)
    X = to_dev(wl.q4_activations(M, K, seed_index=M + 3))
    ref = to_np(q.q4_1_matmul(X, p))
    buf = torch.full((M, N + 3), 7.0, dtype=torch.float32, device=dev)
    q.q4_1_matmul(X, p, out=buf[:, :N])
    got = to_np(buf)
    assert np.array_equal(got[:, :N].view(np.uint32), ref.view(np.uint32))
    assert (got[:, N:] == 7.0).all()
    flat = torch.full((M * N + 1,), 7.0, dtype=torch.float32, device=dev)
    q.q4_1_matmul(X, p, out=flat[1:].view(M, N))
    assert np.array_equal(to_np(flat[1:]).reshape(M, N).view(np.uint32), ref.view(np.uint32))
    assert to_np(flat[:1])[0] == 7.0


def test_q4_matmul_variants_and_determinism(q, orc):
    import torch
    blocks = _blocks(1024, 256, seed=5)
    p = _repack(q, blocks, 1024, 256)
    X16 = wl.q4_activations(16, 1024, seed_index=5)
    X = to_dev(X16)
    a = to_np(q.q4_1_matmul(X, p))
    assert q.last_variant() == "q4_mm16"
    _check(a, orc.q4_1_matmul(X16, blocks, 1024, 256))
    X3 = wl.q4_activations(3, 1024, seed_index=7)
    y3 = to_np(q.q4_1_matmul(to_dev(X3), p))
    assert q.last_variant() == "q4_gemv_m4"
    _check(y3, orc.q4_1_matmul(X3, blocks, 1024, 256))
    b = to_np(q.q4_1_matmul(X, p))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    X20 = wl.q4_activations(20, 1024, seed_index=6)
    y20 = to_np(q.q4_1_matmul(to_dev(X20), p))
    assert q.last_variant() == "q4_mm_m32"
    _check(y20, orc.q4_1_matmul(X20, blocks, 1024, 256))
    # strided X and Y
    Xw = torch.zeros((16, 1024 + 32), dtype=torch.float32, device=torch_dev())
    Xw[:, :1024] = X
    Yw = torch.full((16, 256 + 8), 7.0, dtype=torch.float32, device=torch_dev())
    q.q4_1_matmul(Xw[:, :1024], p, out=Yw[:, :256])
    out = to_np(Yw)
    assert np.array_equal(out[:, :256].view(np.uint32), a.view(np.uint32))
    assert (out[:, 256:] == 7.0).all()


@pytest.mark.parametrize("shape", range(len(wl.Q4_SHAPES)))
@pytest.mark.parametrize("M", wl.Q4_ROWS)
def test_q4_matmul_full_size(q, orc, shape, M):
    """8B-class shapes at M = 1 and 16: full output against the fp64 oracle."""
    K, N = wl.Q4_SHAPES[shape]
    got, ref = _matmul_case(q, orc, M, K, N, seed=shape)
    assert np.isfinite(got).all()


@pytest.mark.parametrize("shape", range(len(wl.Q4_SHAPES)))
@pytest.mark.parametrize("M,variant", [(2, "q4_gemv_m4"), (3, "q4_gemv_m4"), (4, "q4_gemv_m4"),
                                       (20, "q4_mm_m32"), (32, "q4_mm_m32")])
def test_q4_matmul_full_size_other_rows(q, orc, shape, M, variant):
    """The 8B-class shapes through the 2..4-row and 17..32-row kernels: the
    full output against the fp64 oracle at the 1e-5 gate."""
    K, N = wl.Q4_SHAPES[shape]
    got, ref = _matmul_case(q, orc, M, K, N, seed=10 + shape, variant=variant)
    assert np.isfinite(got).all()


# ------------------------------------------------------------ MUL_MAT_ID ---

def _moe_case(q, orc, E, K, N, T, n_used, stride=17, seed=0, ids=None, check="full"):
    g = np.random.default_rng(seed)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    if ids is None:
        ids = np.stack([g.permutation(max(E, stride))[:stride] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    Y = q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used)
    assert q.last_variant() == "q4_moe_m32"
    got = to_np(Y)
    if check == "full":
        ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
        absw = [np.abs(orc.q4_1_decode(experts[e], K, N)) for e in range(E)]
        scale = np.stack([np.stack([np.abs(X[t].astype(np.float64)) @ absw[ids[t, s]] for s in range(n_used)])
                          for t in range(T)])
        _gate(got, ref, scale, K, N)
        for s in range(n_used):
            _gate(got[:, s], ref[:, s], scale[:, s], K, N)
    return got, (experts, X, ids)


def test_moe_small_strided(q, orc):
    got, (experts, X, ids) = _moe_case(q, orc, E=6, K=64, N=24, T=10, n_used=3)
    # the unused tail of each id row changes nothing
    ids2 = ids.copy()
    ids2[:, 3:] = (ids2[:, 3:] + 1) % 6
    buf, estride = q.q4_1_repack_experts(to_dev(experts), 64, 24)
    got2 = to_np(q.q4_1_matmul_id(to_dev(X), buf, 6, 64, 24, estride, to_dev(ids2), 3))
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32))


@pytest.mark.parametrize("E,K,N,T,n_used", [(20, 96, 40, 37, 4), (3, 32, 16, 1, 1), (9, 256, 300, 70, 8),
                                             (128, 64, 48, 64, 8), (700, 32, 16, 1100, 8), (8192, 32, 16, 64, 8)])
def test_moe_shapes(q, orc, E, K, N, T, n_used):
    """(700, ..., 1100, 8): 11 experts per lane of the routing scan and 8800
    pairs, past the 8192 the routing holds in registers; (8192, ...): the
    largest expert count the call accepts (128 KB of routing tables in LDS,
    128 experts per lane of the scan)."""
    _moe_case(q, orc, E, K, N, T, n_used, seed=E + K + N + T)


def test_moe_token_magnitudes(q, orc):
    """Tokens whose magnitudes lie far outside fp16's range (1e-30 .. 1e30,
    mixed in one call): the grouped product's per-token power-of-two scale
    keeps every token, checked token by token, within the 1e-5 gate.  K = 160
    leaves a partial last record."""
    E, K, N, T, n_used = 6, 160, 40, 9, 3
    g = np.random.default_rng(21)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    factors = np.array([1.0, 1e30, 1e-30, 1e-20, 1e20, 3.0e4, 7.5e-6, 1.0, 65504.0], dtype=np.float32)
    X = (wl.normal_f32(g, (T, K)) * factors[:, None]).astype(np.float32)
    ids = np.stack([g.permutation(17)[:17] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    got = to_np(q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used))
    assert np.isfinite(got).all()
    ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
    absw = [np.abs(orc.q4_1_decode(experts[e], K, N)) for e in range(E)]
    for t in range(T):
        scale = np.stack([np.abs(X[t].astype(np.float64)) @ absw[ids[t, s]] for s in range(n_used)])
        _gate(got[t], ref[t], scale, K, N)


def test_moe_unaligned_activations(q, orc):
    """Activation rows one float past a 16-byte boundary (ldx = K + 1): the
    split's scalar-load path gives the same bits as the aligned call."""
    import torch
    E, K, N, T, n_used = 7, 96, 40, 13, 4
    g = np.random.default_rng(8)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(17)[:17] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    a = to_np(q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used))
    Xw = torch.zeros((T, K + 1), dtype=torch.float32, device=torch_dev())
    Xw[:, 1:] = to_dev(X)
    b = to_np(q.q4_1_matmul_id(Xw[:, 1:], buf, E, K, N, estride, to_dev(ids), n_used))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
    absw = [np.abs(orc.q4_1_decode(experts[e], K, N)) for e in range(E)]
    scale = np.stack([np.stack([np.abs(X[t].astype(np.float64)) @ absw[ids[t, s]] for s in range(n_used)])
                      for t in range(T)])
    _gate(b, ref, scale, K, N)


def test_moe_single_expert_takes_all_rows(q, orc):
    """Every pair routed to one expert (many row chunks on one expert): equal
    to the dense product with that expert's weight."""
    E, K, N, T, n_used = 4, 128, 64, 70, 3
    ids = np.full((T, 17), 2, dtype=np.int32)
    got, (experts, X, _) = _moe_case(q, orc, E, K, N, T, n_used, ids=ids, check="none")
    ref = orc.q4_1_matmul(X, experts[2], K, N)
    scale = _abs_scale(orc, X, experts[2], K, N)
    for s in range(n_used):
        _gate(got[:, s], ref, scale, K, N)


def test_moe_out_of_range_id_is_skipped(q, orc):
    """An id outside [0, E) is caught by the routing kernel's own bound check:
    that pair's output row is left untouched, every other pair is correct."""
    import torch
    E, K, N, T, n_used = 5, 64, 32, 6, 2
    g = np.random.default_rng(3)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(17)[:17] % E for _ in range(T)]).astype(np.int32)
    ids[4, 1] = E + 3
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    Y = torch.full((T, n_used, N), -9.0, dtype=torch.float32, device=torch_dev())
    q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used, out=Y)
    got = to_np(Y)
    assert (got[4, 1] == -9.0).all()
    ok = ids.copy()
    ok[4, 1] = 0
    ref = orc.q4_1_matmul_id(X, experts, E, K, N, ok, n_used)
    mask = np.ones((T, n_used), dtype=bool)
    mask[4, 1] = False
    absw = [np.abs(orc.q4_1_decode(experts[e], K, N)) for e in range(E)]
    scale = np.stack([np.stack([np.abs(X[t].astype(np.float64)) @ absw[ok[t, s]] for s in range(n_used)])
                      for t in range(T)])
    _gate(got[mask], ref[mask], scale[mask], K, N)


def test_moe_full_config_sampled(q, orc):
    """128 experts of 2048 x 768 q4_1, 512 tokens, top-8 ids from a stride-17
    view: 24 whole tokens (all slots) against the fp64 oracle plus 4096
    sampled outputs."""
    d = wl.moe_inputs()
    E, K, N = wl.MOE_EXPERTS, wl.MOE_K, wl.MOE_N
    buf, estride = q.q4_1_repack_experts(to_dev(d["experts"]), K, N)
    Y = q.q4_1_matmul_id(to_dev(d["X"]), buf, E, K, N, estride, to_dev(d["ids"]), wl.MOE_USED)
    got = to_np(Y)
    g = np.random.default_rng(11)
    toks = np.sort(g.choice(wl.MOE_TOKENS, 24, replace=False))
    ref = orc.q4_1_matmul_id(d["X"][toks], d["experts"], E, K, N, d["ids"][toks], wl.MOE_USED)
    _check(got[toks], ref)
    it = g.integers(0, wl.MOE_TOKENS, 4096)
    is_ = g.integers(0, wl.MOE_USED, 4096)
    in_ = g.integers(0, N, 4096)
    refs = orc.q4_1_matmul_id_at(d["X"], d["experts"], E, K, N, d["ids"], it, is_, in_)
    _check(got[it, is_, in_], refs)


# ------------------------------------- MUL_MAT_ID, per-slot activations ---

def _moe_slot_case(q, orc, E, K, N, T, n_used, seed=0, pad=0):
    """Per-slot rows X[t, s] (ldx_slot = K + pad) against the fp64 oracle,
    slot by slot."""
    import torch
    g = np.random.default_rng(seed)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, n_used, K))
    ids = np.stack([g.permutation(max(E, 17))[:17] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    Xd = to_dev(X)
    if pad:
        Xw = torch.zeros((T, n_used, K + pad), dtype=torch.float32, device=torch_dev())
        Xw[:, :, :K] = Xd
        Xd = Xw[:, :, :K]
    got = to_np(q.q4_1_matmul_id_per_slot(Xd, buf, E, K, N, estride, to_dev(ids), n_used))
    assert q.last_variant() == "q4_moe_m32"
    ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
    absw = [np.abs(orc.q4_1_decode(experts[e], K, N)) for e in range(E)]
    scale = np.stack([np.stack([np.abs(X[t, s].astype(np.float64)) @ absw[ids[t, s]] for s in range(n_used)])
                      for t in range(T)])
    _gate(got, ref, scale, K, N)
    for s in range(n_used):
        _gate(got[:, s], ref[:, s], scale[:, s], K, N)
    return got, (experts, X, ids, buf, estride)


@pytest.mark.parametrize("E,K,N,T,n_used,pad", [(6, 64, 24, 10, 3, 0), (20, 96, 40, 37, 4, 1), (3, 32, 16, 1, 1, 0),
                                                 (9, 768, 300, 70, 8, 4), (128, 64, 48, 64, 8, 0),
                                                 (700, 32, 16, 1100, 8, 0)])
def test_moe_per_slot_shapes(q, orc, E, K, N, T, n_used, pad):
    """A row per (token, slot): ragged N, a partial last record (K = 96),
    unaligned rows (ldx_slot = K + 1), padded rows (K + 4), one token."""
    _moe_slot_case(q, orc, E, K, N, T, n_used, seed=E + K + N + T, pad=pad)


def test_moe_per_slot_equal_rows_match_shared(q, orc):
    """Every slot row equal to its token's row: the same bits as the shared
    form (each output row depends on its own activation row only)."""
    import torch
    E, K, N, T, n_used = 11, 128, 72, 23, 5
    g = np.random.default_rng(9)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(17)[:17] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    a = to_np(q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used))
    X3 = to_dev(np.repeat(X[:, None, :], n_used, axis=1))
    b = to_np(q.q4_1_matmul_id_per_slot(X3, buf, E, K, N, estride, to_dev(ids), n_used))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # a broadcast view (slot stride 0) is rejected: rows must not overlap
    with pytest.raises(RuntimeError):
        q.q4_1_matmul_id_per_slot(to_dev(X)[:, None, :].expand(T, n_used, K), buf, E, K, N, estride,
                                  to_dev(ids), n_used)


def test_moe_down_config_sampled(q, orc):
    """The down experts: 128 experts of 768 x 2048 q4_1, 512 tokens x top-8
    per-slot rows, ids from a stride-17 view: 16 whole tokens (all slots)
    against the fp64 oracle plus 4096 sampled outputs."""
    d = wl.moe_down_inputs()
    E, K, N = wl.MOE_EXPERTS, wl.MOE_DOWN_K, wl.MOE_DOWN_N
    buf, estride = q.q4_1_repack_experts(to_dev(d["experts"]), K, N)
    Y = q.q4_1_matmul_id_per_slot(to_dev(d["X"]), buf, E, K, N, estride, to_dev(d["ids"]), wl.MOE_USED)
    got = to_np(Y)
    assert np.isfinite(got).all()
    g = np.random.default_rng(12)
    toks = np.sort(g.choice(wl.MOE_TOKENS, 16, replace=False))
    ref = orc.q4_1_matmul_id(d["X"][toks], d["experts"], E, K, N, d["ids"][toks], wl.MOE_USED)
    _check(got[toks], ref)
    it = g.integers(0, wl.MOE_TOKENS, 4096)
    is_ = g.integers(0, wl.MOE_USED, 4096)
    in_ = g.integers(0, N, 4096)
    refs = orc.q4_1_matmul_id_at(d["X"], d["experts"], E, K, N, d["ids"], it, is_, in_, n_used=wl.MOE_USED)
    _check(got[it, is_, in_], refs)


@pytest.mark.parametrize("per_slot", [False, True])
def test_moe_every_chunk_size(q, orc, per_slot):
    """Regression: expert e receives exactly e + 1 (token, slot) pairs, e < 40,
    so the routing table holds full chunks and partial chunks of every size
    from 1 to 32 rows (one or two 16-row tiles); every output row is checked
    against the oracle, in both activation forms."""
    E, K, N, n_used = 40, 256, 300, 4
    T = E * (E + 1) // 2 // n_used
    g = np.random.default_rng(5)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    lst = np.concatenate([np.full(e + 1, e) for e in range(E)])
    g.shuffle(lst)
    ids = np.zeros((T, 17), dtype=np.int32)
    ids[:, :n_used] = lst.reshape(T, n_used)
    ids[:, n_used:] = g.integers(0, E, (T, 17 - n_used))
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    if per_slot:
        X = wl.normal_f32(g, (T, n_used, K))
        got = to_np(q.q4_1_matmul_id_per_slot(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used))
    else:
        X = wl.normal_f32(g, (T, K))
        got = to_np(q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used))
    ref = orc.q4_1_matmul_id(X, experts, E, K, N, ids, n_used)
    for e in range(E):
        sel = ids[:, :n_used] == e
        _check(got[sel], ref[sel])


# --------------------------- q4_1 weights x per-row int8 activations ---

def _q8_case(q, orc, M, K, N, seed, pad=0, **kw):
    """Activations quantised per row on the GPU (bit-exact to the oracle's
    quantiser), then q4_1_matmul_q8 against the oracle's block form."""
    import torch
    blocks = _blocks(K, N, seed, **kw)
    X = wl.q4_activations(M, K, seed_index=seed)
    X[0, :5] = 0.0
    p = _repack(q, blocks, K, N)
    Xq, sa = q.quantize_rows_int8(to_dev(X))
    Qa, so = orc.quantize_rows_int8(X)
    assert np.array_equal(to_np(Xq), Qa)
    if pad:
        Xw = torch.zeros((M, K + pad), dtype=torch.int8, device=torch_dev())
        Xw[:, :K] = Xq
        Xq = Xw[:, :K]
    got = to_np(q.q4_1_matmul_q8(Xq, sa, p))
    assert q.last_variant() == "q4_q8_m16"
    ref = orc.q4_1_matmul_q8(Qa, so, blocks, K, N)
    _gate(got, ref, _abs_scale(orc, Qa.astype(np.float32) * so[:, None], blocks, K, N), K, N)
    return got, ref, (Xq, sa, p)


@pytest.mark.parametrize("M,K,N,pad", [(1, 32, 1, 0), (1, 96, 17, 0), (5, 160, 33, 1), (16, 4096, 64, 0),
                                       (16, 1440, 300, 8), (17, 256, 40, 0), (33, 128, 48, 3), (3, 32 * 45, 20, 0),
                                       (2, 8192, 272, 0)])
def test_q4_q8_shapes(q, orc, M, K, N, pad):
    """Ragged N, a partial last record (K = 96, 160, 1440), one to three
    16-row launches, unaligned activation rows (byte loads), 4, 8 and 16
    wavefronts per strip (2 to 64 records)."""
    _q8_case(q, orc, M, K, N, seed=M + K + N, pad=pad, zero_cols=(3,), zero_scale_blocks=True)


@pytest.mark.parametrize("shape", range(len(wl.Q4_SHAPES)))
@pytest.mark.parametrize("M", wl.Q4_ROWS)
def test_q4_q8_full_size(q, orc, shape, M):
    """8B-class shapes at M = 1 and 16: the full output against the oracle,
    and bitwise equal on a second call."""
    K, N = wl.Q4_SHAPES[shape]
    got, _, (Xq, sa, p) = _q8_case(q, orc, M, K, N, seed=shape)
    again = to_np(q.q4_1_matmul_q8(Xq, sa, p))
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_moe_check_mode_reports_bad_id(q, orc):
    """Check mode: an expert id outside [0, E) makes the call return
    QMM_ERR_INVALID after it ran (that pair's output untouched, the others
    written); the same ids in range pass."""
    import torch
    E, K, N, T, n_used = 5, 64, 32, 6, 2
    g = np.random.default_rng(30)
    experts = np.stack([wl.encode_q4_1(wl.normal_f32(g, (K, N), 0.02)) for _ in range(E)])
    X = wl.normal_f32(g, (T, K))
    ids = np.stack([g.permutation(17)[:17] % E for _ in range(T)]).astype(np.int32)
    buf, estride = q.q4_1_repack_experts(to_dev(experts), K, N)
    q.lib.qmm_set_check(1)
    try:
        q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(ids), n_used)
        bad = ids.copy()
        bad[3, 0] = -1
        Y = torch.full((T, n_used, N), -9.0, dtype=torch.float32, device=torch_dev())
        with pytest.raises(RuntimeError):
            q.q4_1_matmul_id(to_dev(X), buf, E, K, N, estride, to_dev(bad), n_used, out=Y)
        got = to_np(Y)
        assert (got[3, 0] == -9.0).all()
        ok = ids.copy()
        ok[3, 0] = 0
        ref = orc.q4_1_matmul_id(X, experts, E, K, N, ok, n_used)
        mask = np.ones((T, n_used), dtype=bool)
        mask[3, 0] = False
        _check(got[mask], ref[mask])
    finally:
        q.lib.qmm_set_check(0)
