"""Helpers for the GPU parity tests: device placement and readers of the
library's device layouts (test infrastructure; the product never reads its
own layouts back)."""
import numpy as np


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def to_np(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def unpack_int8_codes(packed_bytes: np.ndarray, K: int, N: int):
    """Read codes [K, N] int8, scale [N] f32 and colsum [N] i32 out of a packed
    int8 weight buffer (tile layout: 64 k x 16 n tiles, strip-major; inside a
    tile, 16-byte chunk g*16+c holds k = 16g..16g+15 of column c)."""
    Kp = (K + 63) // 64 * 64
    Np = (N + 15) // 16 * 16
    KT, NS = Kp // 64, Np // 16
    raw = packed_bytes[64:64 + Kp * Np].view(np.int8).reshape(NS, KT, 4, 16, 16)  # s, kt, g, c, j
    codes = raw.transpose(1, 2, 4, 0, 3).reshape(Kp, Np)
    off = 64 + Kp * Np
    scale = packed_bytes[off:off + 4 * Np].view(np.float32)
    colsum = packed_bytes[off + 4 * Np:off + 8 * Np].view(np.int32)
    return codes, scale, colsum, (Kp, Np)


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the float-epilogue parity measure)."""
    denom = np.abs(ref).max()
    return float(np.abs(got.astype(np.float64) - ref).max() / (denom if denom > 0 else 1.0))


def frob_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F (the q4_1 parity measure)."""
    return float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def unpack_q4_records(packed: np.ndarray, K: int, N: int):
    """Read codes [K, N] (uint8 0..15), d bits and m bits [N, K/32] (uint16)
    out of a q4_1 device buffer (records of 4 blocks x 16 columns,
    strip-major after a 64-byte header; see the layout note in the library's
    internal header)."""
    NB = K // 32
    NQ = (NB + 3) // 4
    NS = (N + 15) // 16
    rec = packed[64:64 + NS * NQ * 1280].reshape(NS, NQ, 1280)
    words = rec[:, :, :1024].copy().view(np.uint32).reshape(NS, NQ, 4, 16, 4)  # s, q, g, c, i
    codes = np.zeros((NQ * 4 * 32, NS * 16), dtype=np.uint8)
    for e in range(8):
        pos = 2 * e if e < 4 else 2 * (e - 4) + 1
        nib = ((words >> (4 * pos)) & 15).astype(np.uint8)           # s, q, g, c, i
        # k = 32*(4q+i) + 8g + e ; n = 16s + c
        arr = nib.transpose(1, 4, 2, 0, 3)                            # q, i, g, s, c
        codes.reshape(NQ, 4, 4, 8, NS, 16)[:, :, :, e, :, :] = arr.reshape(NQ, 4, 4, NS, 16)
    sc = rec[:, :, 1024:].copy().view(np.uint16).reshape(NS, NQ, 16, 4, 2)  # s, q, c, i, (d,m)
    dm = sc.transpose(0, 2, 1, 3, 4).reshape(NS * 16, NQ * 4, 2)
    return codes[:K, :N], dm[:N, :NB, 0], dm[:N, :NB, 1]


def canonical_q4_parts(blocks: np.ndarray, K: int, N: int):
    """codes [K, N], d bits, m bits [N, K/32] of canonical blocks [N, K/32, 20]."""
    b = blocks.reshape(N, K // 32, 20)
    d = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    m = b[..., 2].astype(np.uint16) | (b[..., 3].astype(np.uint16) << 8)
    qs = b[..., 4:]
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1)               # N, NB, 32
    return codes.reshape(N, K).T.copy(), d, m
