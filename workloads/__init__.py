"""Seeded synthetic inputs for the quantized projection matmul.

This module only draws inputs (and encodes weights into the q4_1 interchange
format the inputs are given in).  It holds none of the arithmetic under test:
no product, no int8 quantiser, no epilogue, no q4_1 decode.  Both the HIP
path's tests/benchmark and the CPU oracle's tests take their inputs from here.

Shapes follow the pages' workloads:
  * a 16 x 1024 x 1024 uint8 x int8 product with zero points, int32 and fp32
    epilogue ("int8 inference", "Product kernel (Int8Gemm)");
  * the seven Qwen3-0.6B projections, 28 layers ("The ONNX pack", "What the
    graph gives us": 196 projection matmuls);
  * 4096 x 14336 / 14336 x 4096 q4_1 weights (8B-class projections, "Zaya 8B
    Q4NX on the AMD NPU");
  * a 2048-token int8 prefill over the same 8B-class shapes;
  * a 128-expert MUL_MAT_ID with top-8 ids read from a stride-17 view
    ("Zaya 8B Q4NX on the AMD NPU", "The bugs that were the work"), and its
    down experts (768 x 2048), which read a row per (token, slot) ("What's
    next": the per-expert activation form);
  * the Qwen3-0.6B output projection (lm_head: hidden 1024 onto a 151936-word
    vocabulary), one large streaming matmul per decoded token ("The ONNX
    pack", "What works today": the per-token step it is part of).
The pages measure on real checkpoints and text; none are available, so these
seeded draws stand in for them with the stated shapes and distributions.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20261202

QWEN3_0_6B_PROJECTIONS = (
    ("q", 1024, 2048),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 2048, 1024),
    ("gate", 1024, 3072),
    ("up", 1024, 3072),
    ("down", 3072, 1024),
)
QWEN3_0_6B_LAYERS = 28
DECODE_ROWS = (1, 16, 32)

Q4_SHAPES = ((4096, 14336), (14336, 4096))
Q4_ROWS = (1, 16)

PREFILL_M = 2048
PREFILL_SHAPES = ((4096, 4096), (4096, 14336), (14336, 4096))

# the down experts of the same MoE: K x N = 768 x 2048, a row per (token, slot)
MOE_DOWN_K = 768
MOE_DOWN_N = 2048

MOE_EXPERTS = 128
MOE_K = 2048
MOE_N = 768
MOE_TOKENS = 512
MOE_USED = 8
MOE_IDS_STRIDE = 17

LM_HEAD_K = 1024
LM_HEAD_N = 151936
LM_HEAD_ROWS = (1, 16)

Q4_BLOCK = 32
Q4_BLOCK_BYTES = 20


def rng(config: int, shape_index: int = 0) -> np.random.Generator:
    """Generator for one (config, shape) pair: seed = base + 100*config + index."""
    return np.random.Generator(np.random.PCG64(SEED_BASE + 100 * config + shape_index))


# ----------------------------------------------------------------- draws ---

def normal_f32(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform_u8(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)


def uniform_i8(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(-128, 128, size=shape, dtype=np.int64).astype(np.int8)


# ---------------------------------------------------- q4_1 input encoding ---

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the 16-bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


def encode_q4_1(W: np.ndarray) -> np.ndarray:
    """Encode fp32 weights W[K, N] into canonical q4_1 blocks, uint8 [N, K/32, 20].

    Per block of 32 consecutive k of one column: m = bf16(min), d =
    bf16((max - m) / 15), code = clamp(rne((x - m) / d), 0, 15) (0 when d = 0).
    Block bytes: d (bf16, little endian), m (bf16), then 16 code bytes where
    byte j holds element j in the low nibble and element j+16 in the high one.
    This only shapes the inputs; every consumer is given the same codes.
    """
    K, N = W.shape
    assert K % Q4_BLOCK == 0
    nb = K // Q4_BLOCK
    x = np.ascontiguousarray(W.T, dtype=np.float32).reshape(N, nb, Q4_BLOCK)
    lo = x.min(axis=2)
    hi = x.max(axis=2)
    m_bits = f32_to_bf16_bits(lo)
    m = bf16_bits_to_f32(m_bits)
    d_bits = f32_to_bf16_bits((hi - m) / np.float32(15.0))
    d = bf16_bits_to_f32(d_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - m[..., None]) / d[..., None]
    t = np.where(d[..., None] == 0, 0.0, t)
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    out = np.empty((N, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2] = (m_bits & 0xFF).astype(np.uint8)
    out[..., 3] = (m_bits >> 8).astype(np.uint8)
    out[..., 4:] = q[..., :16] | (q[..., 16:] << 4)
    return out


def q4_1_blocks_from_parts(d_bits: np.ndarray, m_bits: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Assemble canonical blocks from explicit parts: d_bits, m_bits [N, nb] uint16,
    codes [N, nb, 32] in 0..15."""
    N, nb = d_bits.shape
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape == (N, nb, 32) and codes.max(initial=0) < 16
    out = np.empty((N, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2] = (m_bits & 0xFF).astype(np.uint8)
    out[..., 3] = (m_bits >> 8).astype(np.uint8)
    out[..., 4:] = codes[..., :16] | (codes[..., 16:] << 4)
    return out


# ------------------------------------------------------------- workloads ---

def int8_product_inputs(M=16, K=1024, N=1024, seed_index=0):
    """uint8 A with zA in [0,255], int8 B with zB in [-128,127], fp32 N(0,1)
    bias, scale 1e-3 (the zero-point product of the int8 docs)."""
    g = rng(1, seed_index)
    A = uniform_u8(g, (M, K))
    zA = int(g.integers(0, 256))
    B = uniform_i8(g, (K, N))
    zB = int(g.integers(-128, 128))
    bias = normal_f32(g, (N,))
    return dict(A=A, zA=zA, B=B, zB=zB, bias=bias, scale=np.float32(1e-3))


def int8_requant_inputs(M=16, K=1024, N=1024, seed_index=50):
    """The same product with an int8 requantised output: int32 bias, output
    zero point in [-128,127], and a multiplier that spreads Y over int8."""
    g = rng(1, seed_index)
    A = uniform_u8(g, (M, K))
    zA = int(g.integers(0, 256))
    B = uniform_i8(g, (K, N))
    zB = int(g.integers(-128, 128))
    # Moments of the uniform draws (not of the data): the bias cancels the
    # expected value of sum_k (a-zA)(b-zB) and the scale maps ~1 std to ~40.
    var_u = (256.0 ** 2 - 1.0) / 12.0
    mean_a, mean_b = 127.5 - zA, -0.5 - zB
    bias_i32 = (np.rint(-K * mean_a * mean_b)
                + g.integers(-5000, 5000, size=N, dtype=np.int64)).astype(np.int32)
    zp_out = int(g.integers(-128, 128))
    std = np.sqrt(K * (var_u + mean_a ** 2) * (var_u + mean_b ** 2))
    scale = np.float32(40.0 / std)
    return dict(A=A, zA=zA, B=B, zB=zB, bias_i32=bias_i32, zp_out=zp_out, scale=scale)


def projection_weight(layer: int, proj_index: int) -> np.ndarray:
    """fp32 N(0, 0.02) weight [K, N] of one Qwen3-0.6B projection."""
    _, K, N = QWEN3_0_6B_PROJECTIONS[proj_index]
    g = rng(2, 1000 + layer * 16 + proj_index)
    return normal_f32(g, (K, N), 0.02)


def projection_activations(M: int, K: int, seed_index: int = 0) -> np.ndarray:
    return normal_f32(rng(2, seed_index), (M, K))


def q4_weight(K: int, N: int, seed_index: int = 0):
    """fp32 N(0,0.02) [K,N] weights and their canonical q4_1 blocks."""
    W = normal_f32(rng(3, 100 + seed_index), (K, N), 0.02)
    return W, encode_q4_1(W)


def q4_activations(M: int, K: int, seed_index: int = 0) -> np.ndarray:
    return normal_f32(rng(3, seed_index), (M, K))


def prefill_inputs(K: int, N: int, M: int = PREFILL_M, seed_index: int = 0):
    """int8 A uniform in [-128,127] (zA = 0), fp32 N(0,0.02) weights for the
    per-column pack, per-row scales U(0.5,1.5)/127."""
    g = rng(4, seed_index)
    A = uniform_i8(g, (M, K))
    W = normal_f32(g, (K, N), 0.02)
    rs = (g.uniform(0.5, 1.5, size=M) / 127.0).astype(np.float32)
    return dict(A=A, W=W, rs=rs)


def lm_head_weight() -> np.ndarray:
    """fp32 N(0, 0.02) output-projection weight [1024, 151936] (622 MB)."""
    return normal_f32(rng(6, 0), (LM_HEAD_K, LM_HEAD_N), 0.02)


def lm_head_activations(M: int, seed_index: int = 0) -> np.ndarray:
    return normal_f32(rng(6, 10 + seed_index), (M, LM_HEAD_K))


def moe_ids(T: int = MOE_TOKENS, n_expert: int = MOE_EXPERTS, stride: int = MOE_IDS_STRIDE,
            seed_index: int = 0) -> np.ndarray:
    """int32 [T, stride]: each row is a prefix of a random permutation of the
    experts (distinct ids); the first n_used of each row are the ones used and
    the tail holds other valid ids, as an argsort's strided view would."""
    g = rng(5, 10 + seed_index)
    ids = np.empty((T, stride), dtype=np.int32)
    for t in range(T):
        ids[t] = g.permutation(n_expert)[:stride]
    return ids


def moe_inputs(n_expert: int = MOE_EXPERTS, K: int = MOE_K, N: int = MOE_N, T: int = MOE_TOKENS,
               seed_index: int = 0):
    """Stacked q4_1 experts [n_expert, N, K/32, 20], activations [T, K], ids [T, 17]."""
    g = rng(5, seed_index)
    experts = np.empty((n_expert, N, K // Q4_BLOCK, Q4_BLOCK_BYTES), dtype=np.uint8)
    for e in range(n_expert):
        experts[e] = encode_q4_1(normal_f32(g, (K, N), 0.02))
    X = normal_f32(g, (T, K))
    ids = moe_ids(T, n_expert, MOE_IDS_STRIDE, seed_index)
    return dict(experts=experts, X=X, ids=ids)


def moe_down_inputs(n_expert: int = MOE_EXPERTS, K: int = MOE_DOWN_K, N: int = MOE_DOWN_N, T: int = MOE_TOKENS,
                    n_used: int = MOE_USED, seed_index: int = 0):
    """Down experts [n_expert, N, K/32, 20], per-slot activations
    [T, n_used, K] (each (token, slot) row its own N(0,1) draw), ids [T, 17]."""
    g = rng(7, seed_index)
    experts = np.empty((n_expert, N, K // Q4_BLOCK, Q4_BLOCK_BYTES), dtype=np.uint8)
    for e in range(n_expert):
        experts[e] = encode_q4_1(normal_f32(g, (K, N), 0.02))
    X = normal_f32(g, (T, n_used, K))
    ids = moe_ids(T, n_expert, MOE_IDS_STRIDE, 100 + seed_index)
    return dict(experts=experts, X=X, ids=ids)
