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
