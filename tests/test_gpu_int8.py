"""GPU parity of the int8 path against the CPU oracle, through the C ABI.

Integer outputs (codes, scales, column sums, int32 accumulators, requantised
int8) must match bit for bit; fp32 epilogue outputs must satisfy
max|dY| <= 2e-6 * max|Y| against the oracle's fp64 value.
"""
import itertools

import numpy as np
import pytest

import workloads as wl
from gpu_util import max_rel_err, to_dev, to_np, torch_dev, unpack_int8_codes

pytestmark = pytest.mark.gpu

F32_TOL = 2e-6


@pytest.fixture(scope="module")
def q():
    import int8_bit_weight_amd as q
    return q


def _packed_np(p):
    return to_np(p.data)


def _check_pack(q, orc, W, raw=False):
    Wd = to_dev(W)
    p = q.pack_b_int8_raw(Wd) if raw else q.pack_b_int8(Wd)
    assert q.last_variant() == ("pack_b_raw" if raw else "pack_b_f32")
    K, N = W.shape
    codes, scale, colsum, (Kp, Np) = unpack_int8_codes(_packed_np(p), K, N)
    Q, s, cs = orc.pack_b_raw(W) if raw else orc.pack_b_int8(W)
    assert np.array_equal(codes[:K, :N], Q)
    assert (codes[K:, :] == 0).all() and (codes[:, N:] == 0).all()
    assert np.array_equal(scale[:N].view(np.uint32), s.view(np.uint32))
    assert np.array_equal(colsum[:N], cs)
    return p, (Q, s, cs)


@pytest.mark.parametrize("K,N", [(1024, 1024), (100, 37), (64, 16), (3072, 1024), (1, 1), (1056, 17)])
def test_pack_b_int8_bit_exact(q, orc, K, N):
    W = wl.normal_f32(np.random.default_rng(K * 7 + N), (K, N), 0.02)
    if N > 3:
        W[:, 2] = 0.0               # all-zero column
        W[5 % K, 3] = 127.0         # scale exactly 1 on column 3
    _check_pack(q, orc, W)


@pytest.mark.parametrize("dtype", [np.int8, np.uint8])
def test_pack_b_raw_bit_exact(q, orc, dtype):
    g = np.random.default_rng(3)
    B = (wl.uniform_u8(g, (200, 40)) if dtype == np.uint8 else wl.uniform_i8(g, (200, 40)))
    _check_pack(q, orc, B, raw=True)


@pytest.mark.parametrize("M,K", [(1, 1024), (16, 1024), (32, 3072), (3, 100), (7, 1)])
def test_quantize_rows_bit_exact(q, orc, M, K):
    X = wl.normal_f32(np.random.default_rng(M * 31 + K), (M, K))
    X[0, :] = 0.0
    if M > 2:
        X[2, K // 2] = 127.0
    Xq, rs = q.quantize_rows_int8(to_dev(X))
    Qo, so = orc.quantize_rows_int8(X)
    assert np.array_equal(to_np(Xq), Qo)
    assert np.array_equal(to_np(rs).view(np.uint32), so.view(np.uint32))


def _gemm_case(q, orc, A, zA, B, zB, *, rs=None, bias=None, scale=1.0, requant=None, expect_variant=None):
    """Run the GPU product with I32 + F32 (+ optional requant) outputs and
    compare with the oracle.  B is a raw int8/uint8 K x N weight."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    dev = torch_dev()
    p = q.pack_b_int8_raw(to_dev(B))
    Ad = to_dev(A)
    y32 = torch.full((M, N), -7, dtype=torch.int32, device=dev)
    yf = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    kw = dict(out_i32=y32, out_f32=yf, scale=scale)
    if rs is not None:
        kw["row_scale"] = to_dev(rs)
    if bias is not None:
        kw["bias_f32"] = to_dev(bias)
    yq = None
    if requant is not None:
        yq = torch.zeros((M, N), dtype=torch.uint8 if requant["u8"] else torch.int8, device=dev)
        kw.update(out_q8=yq, q8_unsigned=requant["u8"], bias_i32=to_dev(requant["bias_i32"]),
                  zp_out=requant["zp_out"])
    q.int8_gemm(Ad, zA, p, zB, **kw)
    if expect_variant:
        assert q.last_variant() == expect_variant
    Y64 = orc.int8_gemm_i64(A, zA, B, zB)
    assert np.abs(Y64).max() < 2 ** 31
    assert np.array_equal(to_np(y32), Y64.astype(np.int32))
    ref = orc.epilogue_f64(Y64, rs, None, scale, bias)
    assert max_rel_err(to_np(yf), ref) <= F32_TOL
    if requant is not None:
        refq = orc.requant(Y64, rs, None, scale, requant["bias_i32"], requant["zp_out"], requant["u8"])
        assert np.array_equal(to_np(yq), refq)
    return y32, yf


def test_int8_product_config(q, orc):
    """uint8 A (zA), int8 B (zB), int32 and fp32 outputs, scale 1e-3 and N(0,1) bias."""
    d = wl.int8_product_inputs()
    _gemm_case(q, orc, d["A"], d["zA"], d["B"], d["zB"], bias=d["bias"], scale=d["scale"],
               expect_variant="int8_decode_m16")


@pytest.mark.parametrize("u8", [False, True])
def test_int8_requant_config(q, orc, u8):
    d = wl.int8_requant_inputs()
    zp = d["zp_out"] + (128 if u8 else 0)
    _gemm_case(q, orc, d["A"], d["zA"], d["B"], d["zB"], scale=d["scale"],
               requant=dict(u8=u8, bias_i32=d["bias_i32"], zp_out=zp))


EDGE_M = [1, 2, 3, 17, 33]
EDGE_K = [32, 64, 96, 1056]
EDGE_N = [1, 15, 17]


@pytest.mark.parametrize("M,K,N", list(itertools.product(EDGE_M, EDGE_K, EDGE_N)))
def test_int8_edge_shapes(q, orc, M, K, N):
    g = np.random.default_rng(M * 1000 + K * 10 + N)
    a_u8, b_u8 = bool(g.integers(0, 2)), bool(g.integers(0, 2))
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_u8(g, (K, N)) if b_u8 else wl.uniform_i8(g, (K, N))
    zA = int(g.integers(0, 256)) - (0 if a_u8 else 128)
    zB = int(g.integers(0, 256)) - (0 if b_u8 else 128)
    rs = g.uniform(0.5, 1.5, M).astype(np.float32)
    bias = wl.normal_f32(g, (N,))
    _gemm_case(q, orc, A, zA, B, zB, rs=rs, bias=bias, scale=np.float32(1e-4),
               expect_variant="int8_decode_m16" if M <= 16 else ("int8_decode_m32" if M <= 32 else None))


@pytest.mark.parametrize("zA,zB", [(0, 0), (255, -128), (0, 127), (128, 0), (255, 127)])
def test_int8_extreme_zero_points(q, orc, zA, zB):
    g = np.random.default_rng(zA * 3 + zB)
    A = wl.uniform_u8(g, (16, 1024))
    A[0, :] = 255
    A[1, :] = 0
    B = wl.uniform_i8(g, (1024, 64))
    B[:, 0] = -128
    B[:, 1] = 127
    _gemm_case(q, orc, A, zA, B, zB)


def test_int8_unaligned_lda_and_strided_outputs(q, orc):
    """A with lda = K + 3 (byte-load path), outputs with ld > N."""
    import torch
    g = np.random.default_rng(77)
    M, K, N = 9, 200, 40
    Afull = wl.uniform_i8(g, (M, K + 3))
    B = wl.uniform_i8(g, (K, N))
    dev = torch_dev()
    Ad = to_dev(Afull)[:, :K]
    p = q.pack_b_int8_raw(to_dev(B))
    y = torch.zeros((M, N + 5), dtype=torch.int32, device=dev)
    q.int8_gemm(Ad, -3, p, 11, out_i32=y[:, :N])
    ref = orc.int8_gemm_i64(np.ascontiguousarray(Afull[:, :K]), -3, B, 11)
    out = to_np(y)
    assert np.array_equal(out[:, :N], ref.astype(np.int32))
    assert (out[:, N:] == 0).all()


# ------------------------------------------ wide decode (many columns) ---

@pytest.mark.parametrize("M,K,N,a_u8,zA,zB", [(1, 1024, 16390, False, 0, 0), (16, 100, 16400, True, 131, -5),
                                              (7, 4096, 16384, False, 0, 7), (32, 2048, 16385, False, -4, 0),
                                              (20, 64, 20000, True, 0, 0), (3, 1056, 16500, True, 255, 127)])
def test_wide_decode_full_compare(q, orc, M, K, N, a_u8, zA, zB):
    """M <= 32 over at least 1024 16-column strips: one wavefront per strip
    over the whole k range.  Ragged N (a partial last strip and a partial last
    workgroup of strips), ragged K, uint8 A, zero points (row sums on the
    MFMA), int32, fp32 and requantised int8 outputs, against the oracle."""
    g = np.random.default_rng(M * 7 + K + N)
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, N))
    rs = g.uniform(0.5, 1.5, M).astype(np.float32)
    bias_i32 = g.integers(-5000, 5000, N).astype(np.int32)
    _gemm_case(q, orc, A, zA, B, zB, rs=rs, bias=wl.normal_f32(g, (N,)), scale=np.float32(3e-5),
               requant=dict(u8=False, bias_i32=bias_i32, zp_out=3),
               expect_variant="int8_decode_wide_m16" if M <= 16 else "int8_decode_wide_m32")


def test_wide_decode_unaligned_a(q, orc):
    """A with lda = K + 3 (byte loads into the LDS copy)."""
    import torch
    g = np.random.default_rng(78)
    M, K, N = 5, 300, 16400
    Afull = wl.uniform_i8(g, (M, K + 3))
    B = wl.uniform_i8(g, (K, N))
    p = q.pack_b_int8_raw(to_dev(B))
    y = torch.zeros((M, N), dtype=torch.int32, device=torch_dev())
    q.int8_gemm(to_dev(Afull)[:, :K], -3, p, 11, out_i32=y)
    assert q.last_variant() == "int8_decode_wide_m16"
    ref = orc.int8_gemm_i64(np.ascontiguousarray(Afull[:, :K]), -3, B, 11)
    assert np.array_equal(to_np(y), ref.astype(np.int32))


def _wide_dynamic_variant(M, K, ldx=None, aligned=True, N=16500):
    """The form int8_gemm_dynamic takes over >= 1024 strips: the quantisation
    inside the wide decode while the rows rounded up to a power of two times
    K stay within 16384 (X 16-byte aligned, K and ldx multiples of 4), its
    persistent form (two workgroups per CU) at M <= 16, K <= 1024 and >= 4096
    strips; else the row quantiser, then the wide decode."""
    mp = 1
    while mp < M:
        mp *= 2
    ldx = K if ldx is None else ldx
    if mp * K <= 16384 and K % 4 == 0 and ldx % 4 == 0 and aligned:
        if M <= 16 and K <= 1024 and (N + 15) // 16 >= 4096:
            return "int8_dynamic_wide_m16p"
        return "int8_dynamic_wide_m16" if M <= 16 else "int8_dynamic_wide_m32"
    return "int8_decode_wide_m16" if M <= 16 else "int8_decode_wide_m32"


@pytest.mark.parametrize("M,K", [(1, 1024), (16, 1024), (32, 1024), (3, 1000), (5, 2048), (9, 1024), (4, 4096),
                                 (1, 4000), (20, 512), (7, 1022)])
def test_wide_decode_dynamic_fused(q, orc, M, K):
    """int8_gemm_dynamic over many columns: with the quantisation inside the
    wide decode (one launch) where the planner takes it, else the row
    quantiser first.  Codes and row scales bit for bit the oracle's, fp32
    outputs bit for bit the two-call form's, int32 the oracle's product."""
    _wide_fused_case(q, orc, M, K, 16500)


@pytest.mark.parametrize("M,K,N", [(1, 1024, 65600), (16, 1024, 65541), (3, 1000, 70000), (9, 512, 65536),
                                   (16, 64, 65536 + 16 * 7 + 3), (5, 1024, 16 * 4096)])
def test_wide_decode_dynamic_persistent(q, orc, M, K, N):
    """The persistent form (>= 4096 strips, M <= 16, K <= 1024): two
    workgroups per CU, each quantising the rows once, each wavefront running its
    strips in turn.  Ragged strip counts per workgroup and wavefront, ragged
    N, K below one tile row (64) and not a multiple of 64; the same bars as
    the one-strip-per-wavefront form."""
    _wide_fused_case(q, orc, M, K, N)


def _wide_fused_case(q, orc, M, K, N):
    import torch
    dev = torch_dev()
    g = np.random.default_rng(M * 13 + K)
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    if M > 2:
        X[1] = 0.0                                        # an all-zero row: scale 0, codes 0
        X[2, K // 3] = 50.0                               # a row maximum inside the row
    p = q.pack_b_int8(to_dev(W))
    Xd = to_dev(X)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    y32 = torch.empty((M, N), dtype=torch.int32, device=dev)
    xq = torch.full((M, K), 99, dtype=torch.int8, device=dev)
    rs = torch.full((M,), -1.0, dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(Xd, p, out_f32=y, out_i32=y32, xq_out=xq, rs_out=rs)
    assert q.last_variant() == _wide_dynamic_variant(M, K, N=N)
    Qa, sa = orc.quantize_rows_int8(X)
    assert np.array_equal(to_np(xq), Qa)
    assert np.array_equal(to_np(rs).view(np.uint32), sa.view(np.uint32))
    Xq2, rs2 = q.quantize_rows_int8(Xd)
    y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(Xq2, 0, p, 0, out_f32=y2, row_scale=rs2)
    assert np.array_equal(to_np(y).view(np.uint32), to_np(y2).view(np.uint32))
    Qb, sb, _ = orc.pack_b_int8(W)
    Y64 = orc.int8_gemm_i64(Qa, 0, Qb, 0)
    assert np.array_equal(to_np(y32), Y64.astype(np.int32))
    assert max_rel_err(to_np(y), orc.epilogue_f64(Y64, sa, sb)) <= F32_TOL


def test_wide_decode_dynamic_unaligned_falls_back(q, orc):
    """X not 16-byte aligned: the row quantiser, then the wide decode, with
    the same bits as the aligned call."""
    import torch
    dev = torch_dev()
    M, K, N = 4, 1024, 16400
    g = np.random.default_rng(77)
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    p = q.pack_b_int8(to_dev(W))
    Xw = torch.zeros((M, K + 1), dtype=torch.float32, device=dev)
    Xw[:, 1:] = to_dev(X)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(Xw[:, 1:], p, out_f32=y)
    assert q.last_variant() == "int8_decode_wide_m16"
    ya = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(to_dev(X), p, out_f32=ya)
    assert q.last_variant() == "int8_dynamic_wide_m16"
    assert torch.equal(y, ya)


@pytest.mark.parametrize("M", [1, 16, 32])
def test_wide_decode_dynamic(q, orc, M):
    """int8_gemm_dynamic over many columns (the quantisation inside the wide
    decode, or in a launch of its own past 16384 row values): the same bits
    as quantize_rows_int8 + int8_gemm, and the oracle's int32 product."""
    import torch
    dev = torch_dev()
    K, N = 1024, 16500
    g = np.random.default_rng(M + 5)
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    p = q.pack_b_int8(to_dev(W))
    Xd = to_dev(X)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    y32 = torch.empty((M, N), dtype=torch.int32, device=dev)
    q.int8_gemm_dynamic(Xd, p, out_f32=y, out_i32=y32)
    assert q.last_variant() == _wide_dynamic_variant(M, K)
    Xq2, rs2 = q.quantize_rows_int8(Xd)
    y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(Xq2, 0, p, 0, out_f32=y2, row_scale=rs2)
    assert np.array_equal(to_np(y).view(np.uint32), to_np(y2).view(np.uint32))
    Qa, sa = orc.quantize_rows_int8(X)
    Qb, sb, _ = orc.pack_b_int8(W)
    Y64 = orc.int8_gemm_i64(Qa, 0, Qb, 0)
    assert np.array_equal(to_np(y32), Y64.astype(np.int32))
    assert max_rel_err(to_np(y), orc.epilogue_f64(Y64, sa, sb)) <= F32_TOL


# ------------------------------------------------ per-axis zero points ---

@pytest.mark.parametrize("M", [1, 16, 32])
def test_wide_and_per_strip_forms_agree_bit_for_bit(q, M):
    """One int8_gemm_dynamic call over 1040 strips (the wide form: one
    wavefront per strip, the quantisation inside or before it) gives, bit for bit, the fp32
    outputs of per-strip calls on column slices of the same weight (the fused
    quantising form at 128 and 96 strips, and the grouped form over the
    slices): per-column packing makes a slice's codes, scales and column sums
    those of the whole, and every form rounds the same epilogue chain."""
    import torch
    dev = torch_dev()
    K, N = 1024, 16640
    g = np.random.default_rng(900 + M)
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    Xd = to_dev(X)
    whole = q.pack_b_int8(to_dev(W))
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(Xd, whole, out_f32=y)
    assert q.last_variant() == _wide_dynamic_variant(M, K)
    cuts = [0, 2048, 3584]
    parts = [q.pack_b_int8(to_dev(np.ascontiguousarray(W[:, a:b]))) for a, b in zip(cuts[:-1], cuts[1:])]
    for (a, b), pk in zip(zip(cuts[:-1], cuts[1:]), parts):
        ys = torch.empty((M, b - a), dtype=torch.float32, device=dev)
        q.int8_gemm_dynamic(Xd, pk, out_f32=ys)
        assert q.last_variant().startswith("int8_dynamic"), q.last_variant()
        assert np.array_equal(to_np(ys).view(np.uint32), to_np(y[:, a:b]).view(np.uint32)), (a, b)
    outs = q.int8_gemm_dynamic_grouped(Xd, parts)
    assert q.last_variant().startswith("int8_dynamic_grouped")
    for (a, b), ys in zip(zip(cuts[:-1], cuts[1:]), outs):
        assert np.array_equal(to_np(ys).view(np.uint32), to_np(y[:, a:b]).view(np.uint32)), (a, b)


def _axis_case(q, orc, M, K, N, a_u8, b_u8, seed, expect_variant, zx=None, zw=None, zy=None):
    """The fused QDQ group with per-axis parameters: int8/uint8 activations
    and weights as given, a zero point and a scale per activation row and per
    weight column, int32 + fp32 + requantised int8 outputs (ep.scale = 1/s_y,
    zp_out = zp_y), against the oracle (integers bit-exact)."""
    import torch
    dev = torch_dev()
    g = np.random.default_rng(seed)
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_u8(g, (K, N)) if b_u8 else wl.uniform_i8(g, (K, N))
    lo_a, lo_b = (0 if a_u8 else -128), (0 if b_u8 else -128)
    zA = (g.integers(lo_a, lo_a + 256, M) if zx is None else np.full(M, zx)).astype(np.int32)
    zB = (g.integers(lo_b, lo_b + 256, N) if zw is None else np.full(N, zw)).astype(np.int32)
    zA[0] = lo_a + 255
    zB[-1] = lo_b
    sx = g.uniform(0.5, 2.0, M).astype(np.float32) / np.float32(127.0)
    sw = g.uniform(0.5, 2.0, N).astype(np.float32) / np.float32(127.0)
    Y64 = orc.int8_gemm_axis_i64(A, zA, B, zB)
    assert np.abs(Y64).max() < 2 ** 31
    sy = np.float32(np.abs(Y64 * sx[:, None].astype(np.float64) * sw[None, :]).max() / 100.0)
    scale = np.float32(1.0) / sy
    zp = int(g.integers(-20, 20)) if zy is None else zy
    p = q.pack_b_int8_raw(to_dev(B))
    y32 = torch.full((M, N), -7, dtype=torch.int32, device=dev)
    yf = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    yq = torch.zeros((M, N), dtype=torch.int8, device=dev)
    q.int8_gemm(to_dev(A), to_dev(zA), p, to_dev(zB), out_i32=y32, out_f32=yf, out_q8=yq, row_scale=to_dev(sx),
                col_scale=to_dev(sw), scale=float(scale), zp_out=zp)
    assert q.last_variant() == expect_variant
    assert np.array_equal(to_np(y32), Y64.astype(np.int32))
    assert max_rel_err(to_np(yf), orc.epilogue_f64(Y64, sx, sw, scale)) <= F32_TOL
    assert np.array_equal(to_np(yq), orc.requant(Y64, sx, sw, scale, None, zp, False))
    return A, zA, B, zB, p


@pytest.mark.parametrize("M,K,N,a_u8,b_u8,variant", [
    (8, 16, 6, False, False, "int8_decode_m16"),          # the pages' proof-graph shape
    (1, 1024, 1024, True, False, "int8_decode_m16"), (16, 1056, 272, False, True, "int8_decode_m16"),
    (32, 3072, 1024, True, True, "int8_decode_m32"), (3, 100, 16400, True, False, "int8_decode_wide_m16"),
    (29, 1024, 16500, False, True, "int8_decode_wide_m32"), (256, 1024, 1024, False, False, "int8_prefill_256x128"),
    (300, 200, 130, True, True, "int8_prefill_256x128"), (300, 256, 16475, True, False, "int8_prefill_256x224")])
def test_per_axis_zero_points(q, orc, M, K, N, a_u8, b_u8, variant):
    _axis_case(q, orc, M, K, N, a_u8, b_u8, seed=M * 3 + K + N, expect_variant=variant)


def test_per_axis_pages_values_and_constant_vectors(q, orc):
    """The pages' per-tensor values zp_x = -40, zp_w = -25, zp_y = -7 on the
    8 x 16 x 6 proof shape, given as constant vectors: the same bits as the
    scalar-zero-point call, and the oracle."""
    import torch
    A, zA, B, zB, p = _axis_case(q, orc, 8, 16, 6, False, False, seed=7, expect_variant="int8_decode_m16",
                                 zx=-40, zw=-25, zy=-7)
    zA[:] = -40
    zB[:] = -25
    dev = torch_dev()
    a = torch.empty((8, 6), dtype=torch.int32, device=dev)
    b = torch.empty((8, 6), dtype=torch.int32, device=dev)
    q.int8_gemm(to_dev(A), to_dev(zA), p, to_dev(zB), out_i32=a)
    q.int8_gemm(to_dev(A), -40, p, -25, out_i32=b)
    assert np.array_equal(to_np(a), to_np(b))
    assert np.array_equal(to_np(a), orc.int8_gemm_i64(A, -40, B, -25).astype(np.int32))


@pytest.mark.parametrize("M,K,N,variant", [(16, 1024, 1024, "int8_decode_m16"), (3, 100, 16400, "int8_decode_wide_m16"),
                                             (300, 200, 130, "int8_prefill_256x128")])
@pytest.mark.parametrize("null_side", ["a", "b"])
def test_per_axis_one_null_vector_uint8(q, orc, M, K, N, variant, null_side):
    """int8_gemm_per_axis with uint8 activations and uint8 weights where one
    zero-point vector is NULL: NULL means zero points of 0 (not the uint8
    midpoint 128), so the result is sum_k A (B - zB[n]) or sum_k (A - zA[m]) B,
    checked bit for bit against the oracle with an all-zero vector."""
    import ctypes
    import torch
    dev = torch_dev()
    g = np.random.default_rng(M + K + N + (null_side == "a"))
    A = wl.uniform_u8(g, (M, K))
    B = wl.uniform_u8(g, (K, N))
    zA = g.integers(0, 256, M).astype(np.int32)
    zB = g.integers(0, 256, N).astype(np.int32)
    if null_side == "a":
        zA[:] = 0
    else:
        zB[:] = 0
    p = q.pack_b_int8_raw(to_dev(B))
    y32 = torch.full((M, N), -7, dtype=torch.int32, device=dev)
    ep = q.qmm_epilogue()
    ep.outputs = q.QMM_OUT_I32
    ep.y_i32, ep.ld_i32 = y32.data_ptr(), y32.stride(0)
    Ad = to_dev(A)
    za = None if null_side == "a" else to_dev(zA)
    zb = None if null_side == "b" else to_dev(zB)
    st = q.lib.int8_gemm_per_axis(Ad.data_ptr(), q.QMM_U8, M, K, K, None if za is None else za.data_ptr(),
                                  p.data.data_ptr(), q.QMM_U8, N, None if zb is None else zb.data_ptr(),
                                  ctypes.byref(ep), None, 0, None)
    assert st == q.QMM_OK
    assert q.last_variant() == variant
    assert np.array_equal(to_np(y32), orc.int8_gemm_axis_i64(A, zA, B, zB).astype(np.int32))


@pytest.mark.parametrize("M,K,N,variant", [(20, 256, 3, "int8_decode_m32"), (300, 128, 5, "int8_prefill_256x128")])
def test_caller_col_scale_with_more_rows_than_columns(q, orc, M, K, N, variant):
    """M > N with a caller's col_scale of exactly N floats and no row scales:
    the kernels read no scale past N (the row-scale fallback load stays on
    element 0), and the fp32 output matches the oracle."""
    import torch
    g = np.random.default_rng(M + N)
    A = wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, N))
    cs = g.uniform(0.5, 2.0, N).astype(np.float32)
    p = q.pack_b_int8_raw(to_dev(B))
    yf = torch.empty((M, N), dtype=torch.float32, device=torch_dev())
    q.int8_gemm(to_dev(A), 0, p, 0, out_f32=yf, col_scale=to_dev(cs), scale=0.01)
    assert q.last_variant() == variant
    Y64 = orc.int8_gemm_i64(A, 0, B, 0)
    assert max_rel_err(to_np(yf), orc.epilogue_f64(Y64, None, cs, 0.01)) <= F32_TOL


@pytest.mark.parametrize("M", [3, 40])
def test_int8_max_k(q, orc, M):
    """The largest K the bound K*255*128 < 2^31 admits that is a multiple of
    64 (65792; 65794 is refused on the host): decode (several rounds of k
    tiles per wavefront) and prefill.  One row of A and one column of B at
    -128 make that output K * 16384 = 1,077,936,128, the largest product sum
    of the bound; the rest is random with zero points."""
    K = 65792
    assert K * 255 * 128 < 2 ** 31 <= (K + 64) * 255 * 128
    g = np.random.default_rng(M)
    A = wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, 40))
    A[1, :] = -128
    B[:, 7] = -128
    y32, _ = _gemm_case(q, orc, A, 0, B, 0, expect_variant="int8_decode_m16" if M <= 16 else "int8_prefill_256x128")
    assert to_np(y32)[1, 7] == K * 16384
    _gemm_case(q, orc, A, 3, B, -5)


def test_int8_empty_is_noop(q):
    import torch
    dev = torch_dev()
    p = q.pack_b_int8_raw(torch.zeros((64, 16), dtype=torch.int8, device=dev))
    y = torch.full((1, 16), 5, dtype=torch.int32, device=dev)
    q.int8_gemm(torch.zeros((0, 64), dtype=torch.int8, device=dev), 0, p, 0, out_i32=y[:0])
    assert (to_np(y) == 5).all()


# ----------------------------------------------- Qwen3-0.6B projections ---

@pytest.mark.parametrize("proj", range(len(wl.QWEN3_0_6B_PROJECTIONS)))
def test_projection_pipeline(q, orc, proj):
    """The decode path as the benchmark runs it: packB of fp32 N(0,0.02)
    weights, per-row quantisation of fp32 N(0,1) activations, int8 product,
    fp32 output -- at M = 1, 16, 32, each step against the oracle."""
    import torch
    name, K, N = wl.QWEN3_0_6B_PROJECTIONS[proj]
    W = wl.projection_weight(0, proj)
    p, (Qb, sb, _) = _check_pack(q, orc, W)
    for M in wl.DECODE_ROWS:
        X = wl.projection_activations(M, K, seed_index=proj * 10 + M)
        Xq, rs = q.quantize_rows_int8(to_dev(X))
        Qa, sa = orc.quantize_rows_int8(X)
        assert np.array_equal(to_np(Xq), Qa)
        assert np.array_equal(to_np(rs).view(np.uint32), sa.view(np.uint32))
        y = torch.empty((M, N), dtype=torch.float32, device=torch_dev())
        y32 = torch.empty((M, N), dtype=torch.int32, device=torch_dev())
        q.int8_gemm(Xq, 0, p, 0, out_f32=y, out_i32=y32, row_scale=rs)
        assert q.last_variant() == ("int8_decode_m16" if M <= 16 else "int8_decode_m32")
        Y64 = orc.int8_gemm_i64(Qa, 0, Qb, 0)
        assert np.array_equal(to_np(y32), Y64.astype(np.int32))
        ref = orc.epilogue_f64(Y64, sa, sb)
        assert max_rel_err(to_np(y), ref) <= F32_TOL, (name, M)


def test_decode_workspace_reuse_and_determinism(q, orc):
    """Back-to-back calls that share one workspace give identical bits (the
    split-K counters are left at zero by every call)."""
    import torch
    d = wl.int8_product_inputs(seed_index=3)
    p = q.pack_b_int8_raw(to_dev(d["B"]))
    A = to_dev(d["A"])
    outs = []
    for _ in range(3):
        yf = torch.empty((16, 1024), dtype=torch.float32, device=torch_dev())
        q.int8_gemm(A, d["zA"], p, d["zB"], out_f32=yf, scale=d["scale"], bias_f32=to_dev(d["bias"]))
        outs.append(to_np(yf))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))


# ------------------------------------------------------------- prefill ---

@pytest.mark.parametrize("M,K,N,zA,zB", [(160, 1056, 272, 0, 0), (200, 96, 40, 5, -7), (33, 64, 17, -128, 127),
                                          (128, 128, 128, 0, 3), (257, 320, 129, 17, 0)])
def test_prefill_full_compare(q, orc, M, K, N, zA, zB):
    g = np.random.default_rng(M + K + N)
    A = wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, N))
    rs = (g.uniform(0.5, 1.5, M) / 127).astype(np.float32)
    _gemm_case(q, orc, A, zA, B, zB, rs=rs, bias=wl.normal_f32(g, (N,)), scale=np.float32(0.01),
               expect_variant="int8_prefill_256x128")


def _prefill_variant(M, K, N):
    """The prefill tile the library picks (aligned A): 256 x 224 where its
    tiles fill the 256 CUs in fewer rounds of work than 256 x 128 ones
    (rounds times strips per tile) and K % 128 == 0."""
    ns, tm = -(-N // 16), -(-M // 256)
    t128, t224 = -(-ns // 8) * tm, -(-ns // 14) * tm
    wide = K % 128 == 0 and -(-t224 // 256) * 14 < -(-t128 // 256) * 8
    return "int8_prefill_256x224" if wide else "int8_prefill_256x128"


@pytest.mark.parametrize("M,K,N,zA,zB,a_u8,req", [
    (256, 128, 32777, 0, 0, False, False),    # one row tile, 2049 strips: ragged last tile
    (300, 256, 16475, 7, -3, False, True),    # two row tiles (ragged M), zero points, int8 out
    (200, 384, 32790, 200, 5, True, True),    # uint8 A, odd pair count (3 pairs)
    (257, 128, 16480, 0, 9, False, False),    # zB only (row sums), one row past a tile
    (256, 128, 32928, 0, 0, False, False)])   # whole tiles only (147 x 224 columns)
def test_prefill_wide_tile(q, orc, M, K, N, zA, zB, a_u8, req):
    """The 256 x 224 tile against the oracle: int32 bit-exact, fp32 within
    2e-6 of max|Y|, int8 requant bit-exact, on shapes where it is picked."""
    assert _prefill_variant(M, K, N) == "int8_prefill_256x224"
    g = np.random.default_rng(M * 7 + K + N)
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, N))
    rs = (g.uniform(0.5, 1.5, M) / 127).astype(np.float32)
    requant = None
    if req:
        requant = dict(u8=False, bias_i32=g.integers(-3000, 3000, N).astype(np.int32), zp_out=3)
    _gemm_case(q, orc, A, zA, B, zB, rs=rs, bias=wl.normal_f32(g, (N,)), scale=np.float32(0.001),
               requant=requant, expect_variant="int8_prefill_256x224")


def test_prefill_wide_tile_fp32_only(q, orc):
    """The fp32-only epilogue of the 256 x 224 tile (no zero points, whole
    tiles: the branch-free store path the M = 2048 prefill takes) and, on a
    ragged shape, its general path, against the oracle."""
    import torch
    dev = torch_dev()
    for M, K, N in ((256, 256, 32928), (260, 128, 16475)):
        assert _prefill_variant(M, K, N) == "int8_prefill_256x224"
        g = np.random.default_rng(M + N)
        A = wl.uniform_i8(g, (M, K))
        B = wl.uniform_i8(g, (K, N))
        rs = (g.uniform(0.5, 1.5, M) / 127).astype(np.float32)
        bias = wl.normal_f32(g, (N,))
        p = q.pack_b_int8_raw(to_dev(B))
        yf = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        q.int8_gemm(to_dev(A), 0, p, 0, out_f32=yf, row_scale=to_dev(rs), bias_f32=to_dev(bias),
                    scale=float(np.float32(0.01)))
        assert q.last_variant() == "int8_prefill_256x224"
        ref = orc.epilogue_f64(orc.int8_gemm_i64(A, 0, B, 0), rs, None, np.float32(0.01), bias)
        assert max_rel_err(to_np(yf), ref) <= F32_TOL


def test_prefill_tile_boundaries(q, orc):
    """Where the 256 x 224 tile does not apply: K % 128 == 64 (a pair count
    that is not whole) keeps the 256 x 128 tile on a shape that would
    otherwise take the wide one; and the dynamic (fp32-activation) form at
    M > 32 quantises, then runs the wide tile, bit for bit the two-call
    result."""
    import torch
    dev = torch_dev()
    g = np.random.default_rng(5)
    M, K, N = 256, 192, 32800
    assert _prefill_variant(M, K, N) == "int8_prefill_256x128" and _prefill_variant(M, 256, N) != "int8_prefill_256x128"
    A = wl.uniform_i8(g, (M, K))
    B = wl.uniform_i8(g, (K, N))
    _gemm_case(q, orc, A, 3, B, -2, rs=(g.uniform(0.5, 1.5, M) / 127).astype(np.float32),
               expect_variant="int8_prefill_256x128")
    M, K, N = 300, 256, 16475
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    p = q.pack_b_int8(to_dev(W))
    Xd = to_dev(X)
    Xq, rs = q.quantize_rows_int8(Xd)
    y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(Xq, 0, p, 0, out_f32=y2, row_scale=rs)
    assert q.last_variant() == "int8_prefill_256x224"
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(Xd, p, out_f32=y)
    assert q.last_variant() == "int8_prefill_256x224"
    assert torch.equal(y, y2)
    Qb, sb, _ = orc.pack_b_int8(W)
    Qa, sa = orc.quantize_rows_int8(X)
    ref = orc.epilogue_f64(orc.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb)
    assert max_rel_err(to_np(y), ref) <= F32_TOL


@pytest.mark.parametrize("shape", range(len(wl.PREFILL_SHAPES)))
def test_prefill_full_size_sampled(q, orc, shape):
    """M = 2048 tokens at the 8B-class shapes: packB of fp32 N(0,0.02)
    weights (bit-exact), int32 and fp32 outputs checked on 4096 sampled
    positions (plus the four corners) against the oracle."""
    import torch
    K, N = wl.PREFILL_SHAPES[shape]
    d = wl.prefill_inputs(K, N, seed_index=shape)
    p, (Qb, sb, _) = _check_pack(q, orc, d["W"])
    dev = torch_dev()
    y32 = torch.empty((wl.PREFILL_M, N), dtype=torch.int32, device=dev)
    yf = torch.empty((wl.PREFILL_M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(to_dev(d["A"]), 0, p, 0, out_i32=y32, out_f32=yf, row_scale=to_dev(d["rs"]))
    assert q.last_variant() == _prefill_variant(wl.PREFILL_M, K, N)
    # the benchmark's form: fp32 output alone (the branch-free epilogue)
    yf1 = torch.empty((wl.PREFILL_M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(to_dev(d["A"]), 0, p, 0, out_f32=yf1, row_scale=to_dev(d["rs"]))
    assert torch.equal(yf1, yf)
    g = np.random.default_rng(99 + shape)
    im = np.concatenate([g.integers(0, wl.PREFILL_M, 4096), [0, 0, wl.PREFILL_M - 1, wl.PREFILL_M - 1]])
    in_ = np.concatenate([g.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    ref = orc.int8_gemm_at(d["A"], 0, Qb, 0, im, in_)
    got32 = to_np(y32)[im, in_]
    assert np.array_equal(got32, ref.astype(np.int32))
    reff = ref.astype(np.float64) * d["rs"][im].astype(np.float64) * sb[in_].astype(np.float64)
    gotf = to_np(yf)[im, in_]
    assert np.abs(gotf - reff).max() <= F32_TOL * np.abs(reff).max()


def test_workspace_shared_across_shapes(q, orc):
    """Regression: one zero-filled workspace reused by decode calls of
    different shapes (different split counts and strip counts)."""
    import torch
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device=torch_dev())
    g = np.random.default_rng(5)
    for (M, K, N) in [(16, 1024, 2048), (1, 1024, 3072), (32, 3072, 1024), (16, 2048, 1024), (1, 64, 4096)]:
        A = wl.uniform_i8(g, (M, K))
        B = wl.uniform_i8(g, (K, N))
        p = q.pack_b_int8_raw(to_dev(B))
        y = torch.empty((M, N), dtype=torch.int32, device=torch_dev())
        q.int8_gemm(to_dev(A), 1, p, -2, out_i32=y, ws=ws)
        assert np.array_equal(to_np(y), orc.int8_gemm_i64(A, 1, B, -2).astype(np.int32)), (M, K, N)
    assert (to_np(ws) == 0).all()


# ------------------------------------------------- dynamic (fused) path ---

def _dynamic_shape(M, K, NS):
    """(row groups, strips per workgroup) of the fused dynamic path, or None
    for two launches.  Fused while some split into 1, 2, 4 or 8 row groups
    keeps E <= 16 and E * K <= 16384 (E = rows per group rounded up to a
    power of two; K <= 4096).  Among those splits and 1, 2 or 4 strips per
    workgroup: the fewest rounds * (rows * K * 4 + S * K * 16) bytes, rounds
    = ceil(workgroups / 256), fewer rows per group on a tie."""
    if K > 4096:
        return None
    best = None
    for g in (1, 2, 4, 8):
        r = -(-M // g)
        e = 1 << max(0, (r - 1).bit_length())
        if e > 16 or e * K > 16384:
            continue
        groups = -(-M // r)
        for s in (1, 2, 4):
            wgs = -(-NS // s) * groups
            key = (-(-wgs // 256) * (r * K * 4 + s * K * 16), e)
            if best is None or key < best[0]:
                best = (key, groups, s)
    return None if best is None else best[1:]


def _dynamic_variant(M, K, NS, grouped=False):
    shape = _dynamic_shape(M, K, NS)
    if shape is None:
        return None
    groups, s = shape
    suffix = "" if s == 1 else "_s%d" % s
    if grouped:
        return "int8_dynamic_grouped" + suffix
    return ("int8_dynamic_m16" if groups == 1 else "int8_dynamic_groups") + suffix


@pytest.mark.parametrize("M,K,N", [(1, 1024, 2048), (16, 1024, 1024), (32, 3072, 1024), (16, 2048, 1024),
                                   (16, 3072, 1024), (1, 3072, 64), (3, 100, 37), (17, 1056, 17), (33, 320, 48),
                                   (80, 256, 130), (16, 64, 16), (32, 1024, 64), (20, 512, 40), (5, 4096, 48),
                                   (2, 2048, 33), (1, 4000, 20), (9, 3000, 16), (4, 4096, 40), (6, 2048, 24),
                                   (32, 1024, 2048), (32, 2048, 1024), (31, 1024, 96), (25, 2048, 40),
                                   (18, 3000, 64), (12, 3072, 48),
                                   # several strips per workgroup, ragged last workgroups
                                   (1, 1024, 6000), (8, 1024, 6144), (24, 1024, 3000), (32, 1024, 4000),
                                   # 4-wavefront workgroups (K <= 1024, S <= 2, >= 192 workgroups), ragged K
                                   (2, 1000, 6144), (1, 1000, 4000), (16, 1000, 4096)])
def test_dynamic_matches_two_step_and_oracle(q, orc, M, K, N):
    """int8_gemm_dynamic == quantize_rows_int8 + int8_gemm bit for bit (fp32
    output, quantised rows, row scales), and the oracle's int32 product."""
    import torch
    dev = torch_dev()
    g = np.random.default_rng(M + K + N)
    W = wl.normal_f32(g, (K, N), 0.02)
    X = wl.normal_f32(g, (M, K))
    X[0] = 0.0
    p = q.pack_b_int8(to_dev(W))
    Xd = to_dev(X)
    Xq2, rs2 = q.quantize_rows_int8(Xd)
    y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    q.int8_gemm(Xq2, 0, p, 0, out_f32=y2, row_scale=rs2)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    y32 = torch.empty((M, N), dtype=torch.int32, device=dev)
    xq = torch.full((M, K), 99, dtype=torch.int8, device=dev)
    rs = torch.full((M,), -1.0, dtype=torch.float32, device=dev)
    q.int8_gemm_dynamic(Xd, p, out_f32=y, out_i32=y32, xq_out=xq, rs_out=rs)
    want = _dynamic_variant(M, K, -(-N // 16))
    if want is not None:
        assert q.last_variant() == want
    elif M <= 16:
        assert q.last_variant() == "int8_decode_m16"
    elif M <= 32:
        assert q.last_variant() == "int8_decode_m32"
    assert np.array_equal(to_np(y).view(np.uint32), to_np(y2).view(np.uint32))
    assert np.array_equal(to_np(xq), to_np(Xq2))
    assert np.array_equal(to_np(rs).view(np.uint32), to_np(rs2).view(np.uint32))
    Qa, sa = orc.quantize_rows_int8(X)
    Qb, sb, _ = orc.pack_b_int8(W)
    Y64 = orc.int8_gemm_i64(Qa, 0, Qb, 0)
    assert np.array_equal(to_np(y32), Y64.astype(np.int32))
    assert max_rel_err(to_np(y), orc.epilogue_f64(Y64, sa, sb)) <= F32_TOL


def _near_tie_rows(M, K, seed):
    """Activation rows whose quotients x/s sit within a few ulps of a
    half-integer (the rounding decisions of rne(x/s)), plus rows with scales
    near the ends of the fp32 range."""
    g = np.random.default_rng(seed)
    X = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        amax = np.float32([1.0, 3.7e-3, 123.456, 2.5e-38, 1.5e38, 7.0][m % 6] * g.uniform(0.5, 2.0))
        s = np.float32(amax / np.float32(127.0))
        j = g.integers(-127, 127, K).astype(np.float32) + np.float32(0.5)
        x = (j * s).astype(np.float32)
        steps = g.integers(-3, 4, K)
        for k in range(K):
            for _ in range(abs(int(steps[k]))):
                x[k] = np.nextafter(x[k], np.float32(np.inf) if steps[k] > 0 else np.float32(-np.inf))
        x = np.clip(x, -amax, amax)
        x[g.integers(0, K)] = amax if m % 2 == 0 else -amax
        X[m] = x
    return X


@pytest.mark.parametrize("M,K", [(1, 1024), (2, 1024), (3, 960), (4, 1024), (7, 96), (8, 1024), (16, 1024),
                                 (32, 1024), (27, 2048)])
def test_dynamic_rounding_near_ties(q, orc, M, K):
    """The fused quantiser's codes equal the oracle's rne(x/s) (IEEE fp32
    division) bit for bit on quotients within ulps of a rounding boundary and
    on scales near both ends of the fp32 range."""
    import torch
    X = _near_tie_rows(M, K, seed=M * 31 + K)
    W = wl.normal_f32(np.random.default_rng(5), (K, 32), 0.02)
    p = q.pack_b_int8(to_dev(W))
    y = torch.empty((M, 32), dtype=torch.float32, device=torch_dev())
    xq = torch.full((M, K), 99, dtype=torch.int8, device=torch_dev())
    rs = torch.full((M,), -1.0, dtype=torch.float32, device=torch_dev())
    q.int8_gemm_dynamic(to_dev(X), p, out_f32=y, xq_out=xq, rs_out=rs)
    assert q.last_variant() == _dynamic_variant(M, K, 2)
    Qa, sa = orc.quantize_rows_int8(X)
    assert np.array_equal(to_np(rs).view(np.uint32), sa.view(np.uint32))
    got = to_np(xq)
    assert np.array_equal(got, Qa), np.argwhere(got != Qa)[:5]
    Xq2, _ = q.quantize_rows_int8(to_dev(X))
    assert np.array_equal(to_np(Xq2), Qa)


@pytest.mark.parametrize("M,N,E", [(1, 64, 1), (4, 2048, 2), (16, 1024, 4), (16, 4096, 8), (32, 4096, 8)])
def test_dynamic_row_max_at_every_lane_position(q, orc, M, N, E):
    """The fused quantiser's row maximum combines every lane and wavefront.
    Row groups of E rows (rounded up to a power of two) keep 64 / E lanes per
    row; each row's largest |x| is placed, over 64 calls, at every offset of a
    64-k tile (so at every lane of its row and every one of the E values a
    lane holds) and in every one of the 16 wavefronts' tiles (values
    elsewhere at most a quarter of it).  The row scales and codes must equal
    the oracle's bit for bit."""
    import torch
    dev = torch_dev()
    K = 1024
    groups, _ = _dynamic_shape(M, K, N // 16)
    rows = -(-M // groups)
    assert 1 << max(0, (rows - 1).bit_length()) == E
    g = np.random.default_rng(300 + M + N)
    p = q.pack_b_int8(to_dev(wl.normal_f32(g, (K, N), 0.02)))
    for trial in range(64):
        X = (g.uniform(-0.25, 0.25, (M, K))).astype(np.float32)
        for m in range(M):
            k = (trial + 11 * m) % 64 + 64 * ((trial + 3 * m) % 16)
            X[m, k] = np.float32(1.0 if (trial + m) % 2 == 0 else -1.0) * np.float32(1.0 + 0.125 * m)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        rs = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        q.int8_gemm_dynamic(to_dev(X), p, out_f32=y, xq_out=xq, rs_out=rs)
        assert q.last_variant() == _dynamic_variant(M, K, N // 16)
        Qa, sa = orc.quantize_rows_int8(X)
        assert np.array_equal(to_np(rs).view(np.uint32), sa.view(np.uint32)), trial
        assert np.array_equal(to_np(xq), Qa), trial


def test_dynamic_without_side_outputs(q, orc):
    import torch
    W = wl.projection_weight(1, 6)
    X = wl.projection_activations(16, W.shape[0], seed_index=3)
    p = q.pack_b_int8(to_dev(W))
    y = torch.empty((16, W.shape[1]), dtype=torch.float32, device=torch_dev())
    q.int8_gemm_dynamic(to_dev(X), p, out_f32=y)
    Qa, sa = orc.quantize_rows_int8(X)
    Qb, sb, _ = orc.pack_b_int8(W)
    assert max_rel_err(to_np(y), orc.epilogue_f64(orc.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb)) <= F32_TOL


def test_packed_header_check_and_check_mode(q):
    """qmm_packed_b_check reads the header back (the layout-version stamp);
    in check mode int8_gemm refuses a buffer whose header does not match
    before launching anything."""
    import ctypes
    import torch
    g = np.random.default_rng(4)
    B = wl.uniform_i8(g, (64, 32))
    p = q.pack_b_int8_raw(to_dev(B))
    ptr = ctypes.c_void_p(p.data.data_ptr())
    assert q.lib.qmm_packed_b_check(ptr, 64, 32, None) == q.QMM_OK
    assert q.lib.qmm_packed_b_check(ptr, 64, 48, None) == q.QMM_ERR_INVALID
    assert q.lib.qmm_packed_b_check(ptr, 128, 32, None) == q.QMM_ERR_INVALID
    A = to_dev(wl.uniform_i8(g, (4, 64)))
    y = torch.zeros((4, 32), dtype=torch.int32, device=torch_dev())
    bad = q.PackedInt8(p.data.clone(), 64, 32, p.bt)
    bad.data[0] ^= 0xFF                     # magic byte
    q.lib.qmm_set_check(1)
    try:
        assert q.lib.qmm_check_enabled() == 1
        q.int8_gemm(A, 0, p, 0, out_i32=y)   # a good buffer passes
        with pytest.raises(RuntimeError):
            q.int8_gemm(A, 0, bad, 0, out_i32=y)
    finally:
        q.lib.qmm_set_check(0)
    assert np.array_equal(to_np(y), _np_product(A, B))


def _np_product(A, B):
    """numpy int64 product of a device int8 A and a host int8 B (zero points 0)."""
    return (to_np(A).astype(np.int64) @ B.astype(np.int64)).astype(np.int32)


# ------------------------------------------------ grouped dynamic decode ---

@pytest.mark.parametrize("M,K,Ns,variant", [
    (1, 1024, (2048, 1024, 1024), None),     # q, k, v
    (16, 1024, (3072, 3072), None),          # gate, up: two row groups, 4 strips per workgroup
    (32, 1024, (2048, 1024, 1024), None),    # four row groups, 4 strips per workgroup
    (1, 1024, (3072, 3072), None),           # 2 strips per workgroup
    (5, 96, (17, 300, 1, 40), None),         # ragged K and N, four items
    (32, 3072, (1024, 16), None),            # eight row groups, a last workgroup of one strip
    (40, 1024, (2048, 1024), None),          # eight row groups of 5 rows
    (32, 1024, (1040, 48, 1008, 17), None),  # items' strips straddle workgroups of 4 strips
    (3, 2048, (4096, 1000), None),           # odd strip count, 2 strips per workgroup
    (32, 2048, (1024,), None),               # one item, 2 strips per workgroup
    (4, 5120, (1024, 48), "int8_decode_m16"),                  # K > 4096: quantise once, then a product each
    (200, 256, (2048, 1024), "int8_prefill_256x128"),          # too many rows: the same two-step form
])
def test_dynamic_grouped_matches_separate_calls(q, orc, M, K, Ns, variant):
    """One grouped launch over weights that share the activations gives, bit
    for bit, the fp32 output of one int8_gemm_dynamic call per weight (with
    and without bias, strided outputs), and the oracle's product of the
    quantised rows and weights."""
    import torch
    dev = torch_dev()
    g = np.random.default_rng(M * 7 + K + sum(Ns))
    X = wl.normal_f32(g, (M, K))
    Ws = [wl.normal_f32(g, (K, n), 0.02) for n in Ns]
    pks = [q.pack_b_int8(to_dev(W)) for W in Ws]
    biases = [to_dev(wl.normal_f32(g, (n,))) if i % 2 == 1 else None for i, n in enumerate(Ns)]
    Xd = to_dev(X)
    outs = [torch.full((M, n + 3), float("nan"), dtype=torch.float32, device=dev)[:, :n] for n in Ns]
    q.int8_gemm_dynamic_grouped(Xd, pks, outs=outs, biases=biases, scale=0.5)
    assert q.last_variant() == (variant or _dynamic_variant(M, K, sum(-(-n // 16) for n in Ns), grouped=True))
    Qa, sa = orc.quantize_rows_int8(X)
    for W, pk, b, Y in zip(Ws, pks, biases, outs):
        n = pk.N
        ref = torch.empty((M, n), dtype=torch.float32, device=dev)
        q.int8_gemm_dynamic(Xd, pk, out_f32=ref, bias_f32=b, scale=0.5)
        assert np.array_equal(to_np(Y).view(np.uint32), to_np(ref).view(np.uint32))
        Qb, sb, _ = orc.pack_b_int8(W)
        want = orc.epilogue_f64(orc.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb, 0.5, None if b is None else to_np(b))
        assert max_rel_err(to_np(Y), want) <= F32_TOL
