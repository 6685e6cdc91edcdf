"""Pins for the oracle's per-column packB and per-row activation quantiser
("The ONNX pack", "The three layers of the pack": int8 with scale = amax/127).
"""
import numpy as np

import workloads as wl
from conftest import load_golden


def test_pack_reconstruction_bound_and_extremes(orc):
    g = np.random.default_rng(11)
    W = wl.normal_f32(g, (333, 45), 0.02)
    Q, s, colsum = orc.pack_b_int8(W)
    amax = np.abs(W).max(axis=0)
    # scale = amax/127 in fp32
    assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32))
    # |q*s - x| <= amax/254 per element (slack for the rounded scale)
    err = np.abs(Q.astype(np.float64) * s.astype(np.float64) - W.astype(np.float64))
    assert (err <= amax.astype(np.float64) / 254 * (1 + 2.0 ** -22)).all()
    # the column max maps to +-127 exactly; codes never reach -128
    idx = np.abs(W).argmax(axis=0)
    assert (np.abs(Q[idx, np.arange(45)]) == 127).all()
    assert Q.min() >= -127 and Q.max() <= 127
    assert np.array_equal(colsum, Q.astype(np.int64).sum(axis=0))


def test_pack_exact_ties_round_to_even(orc):
    """amax = 127 gives scale exactly 1, so codes are rne(x): 2.5 -> 2, 3.5 -> 4."""
    col = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5], dtype=np.float32)
    Q, s, colsum = orc.pack_b_int8(col[:, None])
    assert s[0] == 1.0
    assert Q[:, 0].tolist() == [127, 2, 4, -2, -4, 0, 0, 2, 126]
    assert colsum[0] == sum([127, 2, 4, -2, -4, 0, 0, 2, 126])


def test_pack_zero_column(orc):
    W = np.zeros((64, 3), dtype=np.float32)
    W[:, 1] = 0.5
    Q, s, colsum = orc.pack_b_int8(W)
    assert s[0] == 0 and s[2] == 0 and (Q[:, [0, 2]] == 0).all()
    assert (colsum[[0, 2]] == 0).all()
    assert (Q[:, 1] == 127).all() and colsum[1] == 127 * 64


def test_pack_raw_shift(orc):
    g = np.random.default_rng(12)
    B8 = wl.uniform_u8(g, (40, 9))
    Q, s, colsum = orc.pack_b_raw(B8)
    assert np.array_equal(Q.astype(np.int64), B8.astype(np.int64) - 128)
    assert (s == 1).all() and np.array_equal(colsum, Q.astype(np.int64).sum(0))
    Bs = wl.uniform_i8(g, (40, 9))
    Q, s, colsum = orc.pack_b_raw(Bs)
    assert np.array_equal(Q, Bs) and np.array_equal(colsum, Bs.astype(np.int64).sum(0))


def test_quantize_rows_matches_pack_of_transpose(orc):
    """Per-row quantisation is per-column packB of X^T (same rule, other axis)."""
    g = np.random.default_rng(13)
    X = wl.normal_f32(g, (17, 300))
    X[3] = 0
    Q, s = orc.quantize_rows_int8(X)
    Qt, st, _ = orc.pack_b_int8(np.ascontiguousarray(X.T))
    assert np.array_equal(Q, Qt.T) and np.array_equal(s, st)
    assert s[3] == 0 and (Q[3] == 0).all()


def test_int8_path_error_within_page_gate(orc):
    """The quantised product (per-row activations, per-column weights, int8
    GEMM, dequant) stays inside the page's 2 % gate against fp32."""
    gd = load_golden("quant_error_gate.txt")
    g = np.random.default_rng(14)
    K, N = gd["K"], gd["N"]
    X = wl.normal_f32(g, (64, K))
    W = wl.normal_f32(g, (K, N), 0.02)
    Qa, sa = orc.quantize_rows_int8(X)
    Qb, sb, _ = orc.pack_b_int8(W)
    Y = orc.epilogue_f64(orc.int8_gemm_i64(Qa, 0, Qb, 0), sa, sb)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    rel = np.abs(Y - ref).max() / np.abs(ref).max()
    assert rel < gd["gate"]
    # same order of magnitude as the page's measured 4.8e-3
    assert gd["page_rel_error"] / 10 < rel < gd["page_rel_error"] * 10
