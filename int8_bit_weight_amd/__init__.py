"""Thin Python binding of libqmm.so (the quantized projection matmul for MI355X).

Only argument marshalling lives here: every step of the computation runs in
the library's HIP kernels.  PyTorch supplies device memory and the current
HIP stream.  The binding raises ``ImportError`` if the library has not been
built (``python int8_bit_weight_amd/build.py``); there is no CPU fallback.

Functions carry the names of the C entry points declared in include/qmm.h:
``pack_b_int8``, ``pack_b_int8_raw``, ``quantize_rows_int8``, ``int8_gemm``,
``q4_1_repack``, ``q4_1_matmul``, ``q4_1_matmul_q8``, ``q4_1_matmul_id``,
``q4_1_matmul_id_per_slot``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

# torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch
# first makes libqmm.so bind to that same runtime instead of a second copy
# from /opt/rocm, so both see one device, one set of streams and one heap.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError("libqmm.so is not built; run `python int8_bit_weight_amd/build.py` "
                      "(hipcc, gfx950) first")

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

QMM_OK, QMM_ERR_INVALID, QMM_ERR_UNSUPPORTED, QMM_ERR_WORKSPACE, QMM_ERR_HIP = range(5)
QMM_S8, QMM_U8 = 0, 1
QMM_OUT_I32, QMM_OUT_F32, QMM_OUT_I8, QMM_OUT_U8 = 1, 2, 4, 8
Q4_1_BLOCK_BYTES = 20


class qmm_epilogue(ctypes.Structure):
    _fields_ = [
        ("outputs", ctypes.c_uint32),
        ("y_i32", _P), ("ld_i32", _I64),
        ("y_f32", _P), ("ld_f32", _I64),
        ("y_q8", _P), ("ld_q8", _I64),
        ("row_scale", _P), ("col_scale", _P),
        ("scale", ctypes.c_float),
        ("bias_f32", _P), ("bias_i32", _P),
        ("zp_out", _I32),
    ]


class qmm_dynamic_item(ctypes.Structure):
    _fields_ = [("packedB", _P), ("N", _I64), ("y_f32", _P), ("ld_f32", _I64), ("bias_f32", _P)]


_SIGS = {
    "qmm_pack_b_int8_bytes": (_SZ, [_I64, _I64]),
    "pack_b_int8": (_INT, [_P, _I64, _I64, _I64, _P, _SZ, _P]),
    "pack_b_int8_raw": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _SZ, _P]),
    "qmm_packed_b_check": (_INT, [_P, _I64, _I64, _P]),
    "quantize_rows_int8": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "qmm_int8_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "int8_gemm": (_INT, [_P, _INT, _I64, _I64, _I64, _I32, _P, _INT, _I64, _I32,
                         ctypes.POINTER(qmm_epilogue), _P, _SZ, _P]),
    "int8_gemm_per_axis": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _INT, _I64, _P, _P, _P, _SZ, _P]),
    "qmm_int8_gemm_dynamic_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "int8_gemm_dynamic": (_INT, [_P, _I64, _I64, _I64, _P, _I64, ctypes.POINTER(qmm_epilogue), _P, _I64, _P,
                                 _P, _SZ, _P]),
    "qmm_int8_gemm_dynamic_grouped_workspace_bytes": (_SZ, [_I64, _I64]),
    "int8_gemm_dynamic_grouped": (_INT, [_P, _I64, _I64, _I64, ctypes.POINTER(qmm_dynamic_item), _I64,
                                         ctypes.c_float, _P, _SZ, _P]),
    "qmm_q4_1_packed_bytes": (_SZ, [_I64, _I64]),
    "q4_1_repack": (_INT, [_P, _I64, _I64, _P, _SZ, _P]),
    "qmm_q4_1_matmul_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "q4_1_matmul": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "qmm_q4_1_matmul_id_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64]),
    "q4_1_matmul_id": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _I64, _SZ, _P, _I64, _I64,
                              _P, _I64, _I64, _P, _SZ, _P]),
    "qmm_q4_1_matmul_id_per_slot_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64]),
    "q4_1_matmul_id_per_slot": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _I64, _I64, _SZ, _P, _I64, _I64,
                                       _P, _I64, _I64, _P, _SZ, _P]),
    "q4_1_matmul_q8": (_INT, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "q4_1_matmul_id_noalloc": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _I64, _SZ, _P, _I64, _I64,
                                      _P, _I64, _I64, _P]),
    "qmm_set_check": (None, [_INT]),
    "qmm_check_enabled": (_INT, []),
    "qmm_status_string": (ctypes.c_char_p, [_INT]),
    "qmm_last_hip_error": (_INT, []),
    "qmm_last_variant": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class QmmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib.qmm_status_string(status).decode()
        if status == QMM_ERR_HIP:
            msg += " (hipError %d)" % lib.qmm_last_hip_error()
        super().__init__("%s: %s" % (fn, msg))
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != QMM_OK:
        raise QmmError(fn, status)


def last_variant() -> str:
    return lib.qmm_last_variant().decode()


# -------------------------------------------------------- torch plumbing ---

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a device (cuda) tensor")
    return t.device


_workspaces: dict = {}


def workspace(nbytes: int, device):
    """A zero-filled device workspace of at least nbytes, cached per device.

    The kernels leave the parts they rely on zeroed, so one buffer is reused
    across calls issued on one stream."""
    torch = _torch()
    key = torch.device(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=key)
        _workspaces[key] = ws
    return ws


def _empty_bytes(nbytes: int, device):
    torch = _torch()
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


# ------------------------------------------------------------ int8 path ---

@dataclass
class PackedInt8:
    """A weight packed by pack_b_int8 / pack_b_int8_raw (device bytes + shape)."""
    data: object
    K: int
    N: int
    bt: int = QMM_S8


def pack_b_int8(W, stream=None) -> PackedInt8:
    """Per-column int8 quantisation of fp32 W [K, N] (scale = amax/127)."""
    K, N = W.shape
    nbytes = lib.qmm_pack_b_int8_bytes(K, N)
    out = _empty_bytes(nbytes, _dev(W))
    _check("pack_b_int8", lib.pack_b_int8(_ptr(W), K, N, W.stride(0), _ptr(out), nbytes, _stream(stream)))
    return PackedInt8(out, K, N, QMM_S8)


def pack_b_int8_raw(B, stream=None) -> PackedInt8:
    """Pack an int8 / uint8 weight [K, N] as is (uint8 shifted by 128, scales 1)."""
    torch = _torch()
    K, N = B.shape
    bt = QMM_U8 if B.dtype == torch.uint8 else QMM_S8
    nbytes = lib.qmm_pack_b_int8_bytes(K, N)
    out = _empty_bytes(nbytes, _dev(B))
    _check("pack_b_int8_raw", lib.pack_b_int8_raw(_ptr(B), bt, K, N, B.stride(0), _ptr(out), nbytes,
                                                  _stream(stream)))
    return PackedInt8(out, K, N, bt)


def packed_b_scales(p: PackedInt8):
    """Views of the packed buffer's fp32 column scales and int32 column sums."""
    torch = _torch()
    Np = (p.N + 15) // 16 * 16
    Kp = (p.K + 63) // 64 * 64
    off = 64 + Kp * Np
    scale = p.data[off:off + 4 * Np].view(torch.float32)[: p.N]
    colsum = p.data[off + 4 * Np: off + 8 * Np].view(torch.int32)[: p.N]
    return scale, colsum


def quantize_rows_int8(X, out=None, stream=None):
    """Per-row int8 quantisation of fp32 X [M, K]: returns (Xq int8, row_scale f32).
    `out` may supply preallocated (Xq, row_scale) tensors."""
    torch = _torch()
    M, K = X.shape
    if out is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
        rs = torch.empty((M,), dtype=torch.float32, device=X.device)
    else:
        Xq, rs = out
    _check("quantize_rows_int8", lib.quantize_rows_int8(_ptr(X), M, K, X.stride(0), _ptr(Xq), Xq.stride(0),
                                                        _ptr(rs), _stream(stream)))
    return Xq, rs


def int8_gemm(A, zA: int, packedB: PackedInt8, zB: int = 0, *, out_i32=None, out_f32=None, out_q8=None,
              q8_unsigned: bool = False, row_scale=None, col_scale=None, scale: float = 1.0, bias_f32=None,
              bias_i32=None, zp_out: int = 0, ws=None, stream=None):
    """int8 x int8 -> int32 product with the zero-point correction epilogue.
    zA / zB: scalars, or int32 device vectors (one per row of A / column of the
    weight) for per-axis zero points (int8_gemm_per_axis).

    Writes whichever of out_i32 (int32 [M,N]), out_f32 (fp32 [M,N]) and out_q8
    (int8 or uint8 [M,N]) are given; returns them as a tuple in that order."""
    torch = _torch()
    M, K = A.shape
    if K != packedB.K:
        raise ValueError("A has K=%d, packed weight has K=%d" % (K, packedB.K))
    N = packedB.N
    at = QMM_U8 if A.dtype == torch.uint8 else QMM_S8
    ep = qmm_epilogue()
    outs = 0
    if out_i32 is not None:
        outs |= QMM_OUT_I32
        ep.y_i32, ep.ld_i32 = out_i32.data_ptr(), out_i32.stride(0)
    if out_f32 is not None:
        outs |= QMM_OUT_F32
        ep.y_f32, ep.ld_f32 = out_f32.data_ptr(), out_f32.stride(0)
    if out_q8 is not None:
        outs |= QMM_OUT_U8 if q8_unsigned else QMM_OUT_I8
        ep.y_q8, ep.ld_q8 = out_q8.data_ptr(), out_q8.stride(0)
    ep.outputs = outs
    ep.row_scale = None if row_scale is None else row_scale.data_ptr()
    ep.col_scale = None if col_scale is None else col_scale.data_ptr()
    ep.scale = float(scale)
    ep.bias_f32 = None if bias_f32 is None else bias_f32.data_ptr()
    ep.bias_i32 = None if bias_i32 is None else bias_i32.data_ptr()
    ep.zp_out = int(zp_out)
    need = lib.qmm_int8_gemm_workspace_bytes(M, K, N)
    if ws is None and need > 0:
        ws = workspace(need, A.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    if torch.is_tensor(zA) or torch.is_tensor(zB):
        # per-axis zero points: int32 [M] per activation row, int32 [N] per
        # weight column (a scalar given with a vector becomes a vector)
        def vec(z, n):
            if torch.is_tensor(z):
                assert z.dtype == torch.int32 and z.shape == (n,) and z.is_contiguous()
                return z
            return None if int(z) == 0 else torch.full((n,), int(z), dtype=torch.int32, device=A.device)
        za, zb = vec(zA, M), vec(zB, N)
        _check("int8_gemm_per_axis",
               lib.int8_gemm_per_axis(_ptr(A), at, M, K, A.stride(0), _ptr(za), _ptr(packedB.data), packedB.bt, N,
                                      _ptr(zb), ctypes.byref(ep), _ptr(ws), wsz, _stream(stream)))
        return out_i32, out_f32, out_q8
    _check("int8_gemm", lib.int8_gemm(_ptr(A), at, M, K, A.stride(0), int(zA), _ptr(packedB.data), packedB.bt,
                                      N, int(zB), ctypes.byref(ep), _ptr(ws), wsz, _stream(stream)))
    return out_i32, out_f32, out_q8


def int8_gemm_dynamic_grouped(X, packed, outs=None, biases=None, scale: float = 1.0, ws=None, stream=None):
    """int8_gemm_dynamic over several packed weights that share the fp32
    activations X [M, K] (q/k/v, gate/up), in one launch; fp32 outputs with
    optional per-item biases.  Returns the list of outputs."""
    torch = _torch()
    M, K = X.shape
    n = len(packed)
    if outs is None:
        outs = [torch.empty((M, pk.N), dtype=torch.float32, device=X.device) for pk in packed]
    biases = biases or [None] * n
    items = (qmm_dynamic_item * n)()
    for i, (pk, Y, b) in enumerate(zip(packed, outs, biases)):
        if pk.K != K:
            raise ValueError("item %d has K=%d, X has K=%d" % (i, pk.K, K))
        items[i].packedB = pk.data.data_ptr()
        items[i].N = pk.N
        items[i].y_f32 = Y.data_ptr()
        items[i].ld_f32 = Y.stride(0)
        items[i].bias_f32 = None if b is None else b.data_ptr()
    need = lib.qmm_int8_gemm_dynamic_grouped_workspace_bytes(M, K)
    if ws is None and need > 0:
        ws = workspace(need, X.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check("int8_gemm_dynamic_grouped",
           lib.int8_gemm_dynamic_grouped(_ptr(X), M, K, X.stride(0), items, n, float(scale), _ptr(ws), wsz,
                                         _stream(stream)))
    return outs


def _epilogue(out_i32, out_f32, out_q8, q8_unsigned, row_scale, col_scale, scale, bias_f32, bias_i32, zp_out):
    ep = qmm_epilogue()
    outs = 0
    if out_i32 is not None:
        outs |= QMM_OUT_I32
        ep.y_i32, ep.ld_i32 = out_i32.data_ptr(), out_i32.stride(0)
    if out_f32 is not None:
        outs |= QMM_OUT_F32
        ep.y_f32, ep.ld_f32 = out_f32.data_ptr(), out_f32.stride(0)
    if out_q8 is not None:
        outs |= QMM_OUT_U8 if q8_unsigned else QMM_OUT_I8
        ep.y_q8, ep.ld_q8 = out_q8.data_ptr(), out_q8.stride(0)
    ep.outputs = outs
    ep.row_scale = None if row_scale is None else row_scale.data_ptr()
    ep.col_scale = None if col_scale is None else col_scale.data_ptr()
    ep.scale = float(scale)
    ep.bias_f32 = None if bias_f32 is None else bias_f32.data_ptr()
    ep.bias_i32 = None if bias_i32 is None else bias_i32.data_ptr()
    ep.zp_out = int(zp_out)
    return ep


def int8_gemm_dynamic(X, packedB: PackedInt8, *, out_i32=None, out_f32=None, out_q8=None, q8_unsigned=False,
                      col_scale=None, scale: float = 1.0, bias_f32=None, bias_i32=None, zp_out: int = 0,
                      xq_out=None, rs_out=None, ws=None, stream=None):
    """fp32 activations quantised per row (amax/127) inside the product with a
    weight packed by pack_b_int8; same results as quantize_rows_int8 followed
    by int8_gemm.  Optionally also writes the quantised rows (xq_out) and the
    row scales (rs_out)."""
    M, K = X.shape
    if K != packedB.K or packedB.bt != QMM_S8:
        raise ValueError("weight must be an int8 weight packed for K=%d" % K)
    N = packedB.N
    ep = _epilogue(out_i32, out_f32, out_q8, q8_unsigned, None, col_scale, scale, bias_f32, bias_i32, zp_out)
    need = lib.qmm_int8_gemm_dynamic_workspace_bytes(M, K, N)
    if ws is None and need > 0:
        ws = workspace(need, X.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    ldq = 0 if xq_out is None else xq_out.stride(0)
    _check("int8_gemm_dynamic", lib.int8_gemm_dynamic(_ptr(X), M, K, X.stride(0), _ptr(packedB.data), N,
                                                      ctypes.byref(ep), _ptr(xq_out), ldq, _ptr(rs_out), _ptr(ws),
                                                      wsz, _stream(stream)))
    return out_i32, out_f32, out_q8


# ------------------------------------------------------------ q4_1 path ---

@dataclass
class PackedQ4:
    """A q4_1 weight in the device layout written by q4_1_repack."""
    data: object
    K: int
    N: int


def q4_1_repack(blocks, K: int, N: int, stream=None) -> PackedQ4:
    """Canonical q4_1 blocks (device uint8 [N, K/32, 20]) -> device layout."""
    nbytes = lib.qmm_q4_1_packed_bytes(K, N)
    out = _empty_bytes(nbytes, _dev(blocks))
    _check("q4_1_repack", lib.q4_1_repack(_ptr(blocks), K, N, _ptr(out), nbytes, _stream(stream)))
    return PackedQ4(out, K, N)


def q4_1_matmul(X, W: PackedQ4, out=None, ws=None, stream=None):
    """Y = X @ dequant(W) for fp32 X [M, K]; returns fp32 Y [M, N]."""
    torch = _torch()
    M, K = X.shape
    if K != W.K:
        raise ValueError("X has K=%d, weight has K=%d" % (K, W.K))
    Y = torch.empty((M, W.N), dtype=torch.float32, device=X.device) if out is None else out
    need = lib.qmm_q4_1_matmul_workspace_bytes(M, K, W.N)
    if ws is None and need > 0:
        ws = workspace(need, X.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check("q4_1_matmul", lib.q4_1_matmul(_ptr(X), M, K, X.stride(0), _ptr(W.data), W.N, _ptr(Y), Y.stride(0),
                                          _ptr(ws), wsz, _stream(stream)))
    return Y


def q4_1_repack_experts(blocks, K: int, N: int, stream=None):
    """Stacked canonical experts (device uint8 [E, N, K/32, 20]) -> one device
    buffer holding E repacked experts back to back; returns (buffer, stride)."""
    E = blocks.shape[0]
    stride = lib.qmm_q4_1_packed_bytes(K, N)
    stride = (stride + 255) // 256 * 256
    out = _empty_bytes(stride * E, _dev(blocks))
    for e in range(E):
        _check("q4_1_repack", lib.q4_1_repack(_ptr(blocks[e]), K, N, ctypes.c_void_p(out.data_ptr() + e * stride),
                                              stride, _stream(stream)))
    return out, stride


def q4_1_matmul_q8(Xq, row_scale, W: PackedQ4, out=None, stream=None):
    """Y = diag(row_scale) (Xq @ dequant(W)) for int8 Xq [M, K] (the codes and
    scales of quantize_rows_int8); returns fp32 Y [M, N]."""
    torch = _torch()
    M, K = Xq.shape
    if K != W.K:
        raise ValueError("Xq has K=%d, packed weight has K=%d" % (K, W.K))
    assert Xq.dtype == torch.int8 and Xq.stride(1) == 1
    Y = torch.empty((M, W.N), dtype=torch.float32, device=Xq.device) if out is None else out
    _check("q4_1_matmul_q8", lib.q4_1_matmul_q8(_ptr(Xq), _ptr(row_scale), M, K, Xq.stride(0), _ptr(W.data), W.N,
                                                _ptr(Y), Y.stride(0), _stream(stream)))
    return Y


def q4_1_matmul_id(X, experts, n_expert: int, K: int, N: int, expert_stride: int, ids, n_used: int, out=None,
                   ws=None, stream=None):
    """MUL_MAT_ID: Y[t, s] = X[t] @ W_{ids[t, s]} for the first n_used ids of
    each row of the int32 id tensor (its row stride is read from the tensor)."""
    torch = _torch()
    T = X.shape[0]
    Y = torch.empty((T, n_used, N), dtype=torch.float32, device=X.device) if out is None else out
    need = lib.qmm_q4_1_matmul_id_workspace_bytes(T, n_used, n_expert, K, N)
    if ws is None and need > 0:
        ws = workspace(need, X.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check("q4_1_matmul_id", lib.q4_1_matmul_id(_ptr(X), T, K, X.stride(0), _ptr(experts), n_expert, N,
                                                expert_stride, _ptr(ids), ids.stride(0), n_used, _ptr(Y),
                                                Y.stride(1), Y.stride(0), _ptr(ws), wsz, _stream(stream)))
    return Y


def q4_1_matmul_id_noalloc(X, experts, n_expert: int, K: int, N: int, expert_stride: int, ids, n_used: int,
                           out=None, stream=None):
    """q4_1_matmul_id without a workspace: the library's own per-GPU scratch
    array holds the routing tables and split activations (calls that overlap
    on one GPU race)."""
    torch = _torch()
    T = X.shape[0]
    Y = torch.empty((T, n_used, N), dtype=torch.float32, device=X.device) if out is None else out
    _check("q4_1_matmul_id_noalloc",
           lib.q4_1_matmul_id_noalloc(_ptr(X), T, K, X.stride(0), _ptr(experts), n_expert, N, expert_stride,
                                      _ptr(ids), ids.stride(0), n_used, _ptr(Y), Y.stride(1), Y.stride(0),
                                      _stream(stream)))
    return Y


def q4_1_matmul_id_per_slot(X, experts, n_expert: int, K: int, N: int, expert_stride: int, ids, n_used: int,
                            out=None, ws=None, stream=None):
    """MUL_MAT_ID with a row per (token, slot): Y[t, s] = X[t, s] @ W_{ids[t, s]}
    for fp32 X [T, n_used, K] (unit stride along K)."""
    torch = _torch()
    T = X.shape[0]
    assert X.dim() == 3 and X.shape[1] == n_used and X.shape[2] == K and X.stride(2) == 1
    Y = torch.empty((T, n_used, N), dtype=torch.float32, device=X.device) if out is None else out
    need = lib.qmm_q4_1_matmul_id_per_slot_workspace_bytes(T, n_used, n_expert, K, N)
    if ws is None and need > 0:
        ws = workspace(need, X.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check("q4_1_matmul_id_per_slot",
           lib.q4_1_matmul_id_per_slot(_ptr(X), T, K, X.stride(1), X.stride(0), _ptr(experts), n_expert, N,
                                       expert_stride, _ptr(ids), ids.stride(0), n_used, _ptr(Y), Y.stride(1),
                                       Y.stride(0), _ptr(ws), wsz, _stream(stream)))
    return Y
