"""Pins for the oracle's int8 product and epilogues (CPU only).

Each test ties the oracle to something other than itself: a textbook routine
(numpy int64 matmul), the pages' expanded zero-point identities computed by a
different route, brute force over tiny shapes, a value the pages print, or a
tie case whose rounding the pages fix.
"""
import itertools

import numpy as np
import pytest

import workloads as wl
from conftest import load_golden


def _rand_operands(g, M, K, N, a_u8, b_u8):
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_u8(g, (K, N)) if b_u8 else wl.uniform_i8(g, (K, N))
    return A, B


def test_zero_zero_points_is_plain_matmul(orc):
    g = np.random.default_rng(1)
    for a_u8, b_u8 in itertools.product([0, 1], repeat=2):
        A, B = _rand_operands(g, 7, 53, 19, a_u8, b_u8)
        ref = A.astype(np.int64) @ B.astype(np.int64)
        assert np.array_equal(orc.int8_gemm_i64(A, 0, B, 0), ref)


@pytest.mark.parametrize("a_u8,b_u8", list(itertools.product([0, 1], repeat=2)))
def test_shifted_correction_identity(orc, a_u8, b_u8):
    """"int8 inference", "Product kernel": S on operands shifted into the int8
    range, then Y = S - zA'*colSum[n] - zB'*(rowSum[m] - K*zA') must equal the
    direct definition, including extreme zero points."""
    g = np.random.default_rng(2 + 2 * a_u8 + b_u8)
    M, K, N = 5, 77, 11
    A, B = _rand_operands(g, M, K, N, a_u8, b_u8)
    za_range = [0, 255, 128, 37] if a_u8 else [-128, 127, 0, -41]
    zb_range = [0, 255, 128, 201] if b_u8 else [-128, 127, 0, 19]
    Ap = A.astype(np.int64) - (128 if a_u8 else 0)
    Bp = B.astype(np.int64) - (128 if b_u8 else 0)
    S = Ap @ Bp
    col = Bp.sum(axis=0)
    row = Ap.sum(axis=1)
    for zA, zB in itertools.product(za_range, zb_range):
        zAp = zA - (128 if a_u8 else 0)
        zBp = zB - (128 if b_u8 else 0)
        Y = S - zAp * col[None, :] - zBp * (row[:, None] - K * zAp)
        assert np.array_equal(orc.int8_gemm_i64(A, zA, B, zB), Y), (zA, zB)


def test_expanded_zero_point_identity(orc):
    """"The ONNX pack", "What works today": sum (a-zx)(w-zw) = sum aw - zx*sum w
    - zw*sum a + K*zx*zw, on the unshifted values."""
    g = np.random.default_rng(9)
    A, B = _rand_operands(g, 4, 64, 6, 0, 0)
    a = A.astype(np.int64)
    w = B.astype(np.int64)
    for zx, zw in [(-40, -25), (0, 0), (127, -128), (-128, 127)]:
        ref = a @ w - zx * w.sum(0)[None, :] - zw * a.sum(1)[:, None] + 64 * zx * zw
        assert np.array_equal(orc.int8_gemm_i64(A, zx, B, zw), ref)


def test_brute_force_tiny_shapes(orc):
    """Every M, N, K in {1,2,3} over small value sets including the extremes;
    the expected value is a pure-Python loop."""
    vals_u8 = [0, 1, 127, 128, 254, 255]
    vals_i8 = [-128, -1, 0, 1, 127]
    g = np.random.default_rng(3)
    for M, K, N in itertools.product([1, 2, 3], repeat=3):
        for a_u8, b_u8 in itertools.product([0, 1], repeat=2):
            va = vals_u8 if a_u8 else vals_i8
            vb = vals_u8 if b_u8 else vals_i8
            A = np.array(g.choice(va, size=(M, K)), dtype=np.uint8 if a_u8 else np.int8)
            B = np.array(g.choice(vb, size=(K, N)), dtype=np.uint8 if b_u8 else np.int8)
            zA = int(g.choice(va))
            zB = int(g.choice(vb))
            got = orc.int8_gemm_i64(A, zA, B, zB)
            for m in range(M):
                for n in range(N):
                    s = 0
                    for k in range(K):
                        s += (int(A[m, k]) - zA) * (int(B[k, n]) - zB)
                    assert got[m, n] == s


def test_sampled_matches_full(orc):
    d = wl.int8_product_inputs(M=8, K=96, N=40)
    Y = orc.int8_gemm_i64(d["A"], d["zA"], d["B"], d["zB"])
    im = np.array([0, 7, 3, 5])
    in_ = np.array([0, 39, 17, 2])
    assert np.array_equal(orc.int8_gemm_at(d["A"], d["zA"], d["B"], d["zB"], im, in_), Y[im, in_])


def test_int32_bound(orc):
    gd = load_golden("int8_bound.txt")
    assert gd["bound_factor"] == 255 * 128
    assert orc.int8_bound_ok(gd["k_about"])
    assert orc.int8_bound_ok(gd["k_largest_model"])
    kmax = (2 ** 31 - 1) // gd["bound_factor"]
    assert orc.int8_bound_ok(kmax) and not orc.int8_bound_ok(kmax + 1)
    for K in (1024, 2048, 3072, 4096, 14336):   # every K of the workloads
        assert orc.int8_bound_ok(K)


# ------------------------------------------------------------ epilogues ---

def test_f64_epilogue_closed_form(orc):
    Y = np.array([[1000, -2000], [0, 7]], dtype=np.int64)
    rs = np.array([0.5, 2.0], dtype=np.float32)
    cs = np.array([0.25, 4.0], dtype=np.float32)
    bias = np.array([1.0, -1.0], dtype=np.float32)
    out = orc.epilogue_f64(Y, rs, cs, 1e-3, bias)
    s = float(np.float32(1e-3))
    exp = np.array([[1000 * 0.5 * 0.25 * s + 1, -2000 * 0.5 * 4 * s - 1],
                    [1.0, 7 * 2 * 4 * s - 1]])
    assert np.allclose(out, exp, rtol=0, atol=1e-12)
    assert np.array_equal(orc.epilogue_f64(Y), Y.astype(np.float64))


def _mult_for(acc, target):
    """Search fp32 multipliers near target/acc for one whose fp32 product with
    fp32(acc) is the fp32 value nearest `target` (numpy fp32 arithmetic)."""
    want = np.float32(target)
    up = down = np.float32(target / acc)
    for _ in range(256):
        for m in (up, down):
            if np.float32(np.float32(acc) * m) == want:
                return m
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
    raise AssertionError("no multiplier found")


def test_requant_page_tie_example(orc):
    """The worked example: accumulator -3090 whose scaled value is -3.499998
    rounds to -3; a value of exactly -3.5 rounds half to even to -4.  With one
    fp32 multiply, fp32(-3090) * m never lands exactly on -3.5 for m near
    3.5/3090, so the exact tie is shown with accumulator -7 and m = 0.5."""
    gd = load_golden("requant_tie.txt")
    acc = gd["accumulator"]
    mult = _mult_for(acc, gd["near_tie_value"])
    assert orc.requant(np.array([[acc]], dtype=np.int64), scale=mult)[0, 0] == gd["near_tie_result"]
    with pytest.raises(AssertionError):
        _mult_for(acc, gd["exact_tie_value"])
    assert np.float32(-7) * np.float32(0.5) == np.float32(gd["exact_tie_value"])
    assert orc.requant(np.array([[-7]], dtype=np.int64), scale=0.5)[0, 0] == gd["exact_tie_result"]


def test_requant_ties_to_even_and_zero_point_after_rounding(orc):
    Y = np.array([[1, 3, 5, -1, -3, -5, 7]], dtype=np.int64)
    # mult 0.5 makes every product an exact tie: 0.5 1.5 2.5 -0.5 -1.5 -2.5 3.5
    out = orc.requant(Y, scale=0.5)
    assert out.tolist() == [[0, 2, 2, 0, -2, -2, 4]]
    # output zero point after rounding: rne(2.5) + 1 = 3, not rne(3.5) = 4
    out = orc.requant(np.array([[5]], dtype=np.int64), scale=0.5, zp_out=1)
    assert out[0, 0] == 3
    # int32 bias enters before the multiply
    out = orc.requant(np.array([[3]], dtype=np.int64), scale=0.5, bias_i32=np.array([2]))
    assert out[0, 0] == 2   # (3+2)*0.5 = 2.5 -> 2


def test_requant_clamps_and_u8(orc):
    Y = np.array([[10 ** 6, -10 ** 6, 0]], dtype=np.int64)
    assert orc.requant(Y, scale=1.0).tolist() == [[127, -128, 0]]
    out = orc.requant(Y, scale=1.0, zp_out=128, out_u8=True)
    assert out.dtype == np.uint8 and out.tolist() == [[255, 0, 128]]
    with pytest.raises(OverflowError):
        orc.requant(np.array([[2 ** 31]], dtype=np.int64), scale=1.0)


def test_requant_scales_fold_in_fp32_order(orc):
    """mult = fl32(fl32(rs*cs)*scale), then one fp32 multiply: checked against
    the same chain evaluated with numpy fp32 scalars on random data."""
    g = np.random.default_rng(5)
    Y = g.integers(-10 ** 6, 10 ** 6, size=(6, 9)).astype(np.int64)
    rs = g.uniform(0.1, 2, 6).astype(np.float32)
    cs = g.uniform(0.1, 2, 9).astype(np.float32)
    scale = np.float32(3e-5)
    out = orc.requant(Y, rs, cs, scale, zp_out=-7)
    for m in range(6):
        for n in range(9):
            mult = np.float32(np.float32(rs[m] * cs[n]) * scale)
            v = np.float32(np.float32(Y[m, n]) * mult)
            exp = int(np.clip(np.rint(v) - 7, -128, 127))
            assert out[m, n] == exp


# ---------------------------------------------- per-axis zero points ---
# "The ONNX pack", "What works today": a zero point per activation row and
# one per weight column, on the same axes as the per-axis scales.

@pytest.mark.parametrize("a_u8,b_u8", [(False, False), (True, False), (False, True), (True, True)])
def test_axis_zero_points_against_numpy(orc, a_u8, b_u8):
    """numpy int64 product of the explicitly shifted matrices."""
    g = np.random.default_rng(61 + 2 * a_u8 + b_u8)
    M, K, N = 9, 70, 13
    A = wl.uniform_u8(g, (M, K)) if a_u8 else wl.uniform_i8(g, (M, K))
    B = wl.uniform_u8(g, (K, N)) if b_u8 else wl.uniform_i8(g, (K, N))
    lo_a, lo_b = (0 if a_u8 else -128), (0 if b_u8 else -128)
    zA = g.integers(lo_a, lo_a + 256, M).astype(np.int32)
    zB = g.integers(lo_b, lo_b + 256, N).astype(np.int32)
    zA[0], zB[0] = lo_a, lo_b + 255            # range ends
    ref = (A.astype(np.int64) - zA[:, None]) @ (B.astype(np.int64) - zB[None, :])
    assert np.array_equal(orc.int8_gemm_axis_i64(A, zA, B, zB), ref)


def test_axis_zero_points_reduce_to_scalar(orc):
    """Constant vectors give the per-tensor product (pinned above)."""
    g = np.random.default_rng(62)
    A = wl.uniform_u8(g, (5, 33))
    B = wl.uniform_i8(g, (33, 7))
    Y = orc.int8_gemm_axis_i64(A, np.full(5, 200, np.int32), B, np.full(7, -25, np.int32))
    assert np.array_equal(Y, orc.int8_gemm_i64(A, 200, B, -25))


def test_axis_zero_points_expanded_identity_brute_force(orc):
    """The page's expansion sum a*w - zx*sum w - zw*sum a + K*zx*zw, evaluated
    with Python integers over every entry of tiny shapes with extreme
    values; each row and column its own zero point."""
    vals = [-128, -1, 0, 1, 127]
    for M, K, N in [(1, 1, 1), (2, 3, 2), (3, 2, 3)]:
        g = np.random.default_rng(M * 100 + K * 10 + N)
        A = g.choice(vals, (M, K)).astype(np.int8)
        B = g.choice(vals, (K, N)).astype(np.int8)
        zA = g.choice(vals, M).astype(np.int32)
        zB = g.choice(vals, N).astype(np.int32)
        Y = orc.int8_gemm_axis_i64(A, zA, B, zB)
        for m in range(M):
            for n in range(N):
                a = [int(v) for v in A[m]]
                w = [int(B[k, n]) for k in range(K)]
                zx, zw = int(zA[m]), int(zB[n])
                want = sum(x * y for x, y in zip(a, w)) - zx * sum(w) - zw * sum(a) + K * zx * zw
                assert Y[m, n] == want
