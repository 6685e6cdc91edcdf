"""CPU oracle for the quantized projection matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.

The arithmetic lives in ``oracle.c`` (plain C, int64 / fp64, built with gcc
``-O2 -fopenmp -ffp-contract=off``, no fast-math).  This module only builds
that file and marshals numpy arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_F32 = ctypes.c_float


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_int8_bound_ok": (_INT, [_I64]),
        "oracle_int8_gemm_i64": (None, [_P, _INT, _I64, _I64, _I64, _I32, _P, _INT, _I64, _I64, _I32, _P, _I64]),
        "oracle_int8_gemm_axis_i64": (None, [_P, _INT, _I64, _I64, _I64, _P, _P, _INT, _I64, _I64, _P, _P, _I64]),
        "oracle_int8_gemm_at": (None, [_P, _INT, _I64, _I64, _I32, _P, _INT, _I64, _I32, _P, _P, _I64, _P]),
        "oracle_epilogue_f64": (None, [_P, _I64, _I64, _I64, _P, _P, _F32, _P, _P]),
        "oracle_requant": (_INT, [_P, _I64, _I64, _I64, _P, _P, _F32, _P, _I32, _INT, _P]),
        "oracle_pack_b_int8": (None, [_P, _I64, _I64, _I64, _P, _P, _P]),
        "oracle_pack_b_raw": (None, [_P, _INT, _I64, _I64, _I64, _P, _P, _P]),
        "oracle_quantize_rows_int8": (None, [_P, _I64, _I64, _I64, _P, _P]),
        "oracle_q4_1_decode": (None, [_P, _I64, _I64, _P]),
        "oracle_q4_1_matmul": (None, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64]),
        "oracle_q4_1_matmul_at": (None, [_P, _I64, _I64, _P, _P, _P, _I64, _P]),
        "oracle_q4_1_matmul_q8": (None, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _I64]),
        "oracle_q4_1_matmul_id": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _I64,
                                         _I64]),
        "oracle_q4_1_matmul_id_at": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _P, _I64, _P]),
        "oracle_num_threads": (_INT, []),
        "oracle_set_num_threads": (None, [_INT]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 1, "oracle arrays must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i8kind(a: np.ndarray) -> int:
    if a.dtype == np.uint8:
        return 1
    if a.dtype == np.int8:
        return 0
    raise TypeError("expected int8 or uint8, got %s" % a.dtype)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use (timing only)."""
    _load().oracle_set_num_threads(int(n))


def int8_bound_ok(K: int) -> bool:
    return bool(_load().oracle_int8_bound_ok(K))


def int8_gemm_i64(A: np.ndarray, zA: int, B: np.ndarray, zB: int) -> np.ndarray:
    """Y[m,n] = sum_k (A[m,k]-zA)(B[k,n]-zB) as int64 (naive)."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    Y = np.empty((M, N), dtype=np.int64)
    _load().oracle_int8_gemm_i64(_ptr(A), _i8kind(A), M, K, K, zA, _ptr(B), _i8kind(B), N, N, zB, _ptr(Y), N)
    return Y


def int8_gemm_axis_i64(A: np.ndarray, zA, B: np.ndarray, zB) -> np.ndarray:
    """Per-axis zero points: Y[m,n] = sum_k (A[m,k]-zA[m])(B[k,n]-zB[n]) as
    int64 (naive); zA [M] and zB [N] int32."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    zA = np.ascontiguousarray(zA, dtype=np.int32)
    zB = np.ascontiguousarray(zB, dtype=np.int32)
    assert zA.shape == (M,) and zB.shape == (N,)
    Y = np.empty((M, N), dtype=np.int64)
    _load().oracle_int8_gemm_axis_i64(_ptr(A), _i8kind(A), M, K, K, _ptr(zA), _ptr(B), _i8kind(B), N, N, _ptr(zB),
                                      _ptr(Y), N)
    return Y


def int8_gemm_at(A: np.ndarray, zA: int, B: np.ndarray, zB: int, im, in_) -> np.ndarray:
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    _, N = B.shape
    im = np.ascontiguousarray(im, dtype=np.int64)
    in_ = np.ascontiguousarray(in_, dtype=np.int64)
    assert im.shape == in_.shape
    assert (im >= 0).all() and (im < M).all() and (in_ >= 0).all() and (in_ < N).all()
    out = np.empty(im.shape, dtype=np.int64)
    _load().oracle_int8_gemm_at(_ptr(A), _i8kind(A), K, K, zA, _ptr(B), _i8kind(B), N, zB,
                                _ptr(im), _ptr(in_), im.size, _ptr(out))
    return out


def epilogue_f64(Y: np.ndarray, rs=None, cs=None, scale: float = 1.0, bias=None) -> np.ndarray:
    Y = np.ascontiguousarray(Y, dtype=np.int64)
    M, N = Y.shape
    rs = None if rs is None else np.ascontiguousarray(rs, dtype=np.float32)
    cs = None if cs is None else np.ascontiguousarray(cs, dtype=np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_epilogue_f64(_ptr(Y), M, N, N, _ptr(rs), _ptr(cs), float(scale), _ptr(bias), _ptr(out))
    return out


def requant(Y: np.ndarray, rs=None, cs=None, scale: float = 1.0, bias_i32=None,
            zp_out: int = 0, out_u8: bool = False) -> np.ndarray:
    Y = np.ascontiguousarray(Y, dtype=np.int64)
    M, N = Y.shape
    rs = None if rs is None else np.ascontiguousarray(rs, dtype=np.float32)
    cs = None if cs is None else np.ascontiguousarray(cs, dtype=np.float32)
    bias_i32 = None if bias_i32 is None else np.ascontiguousarray(bias_i32, dtype=np.int32)
    out = np.empty((M, N), dtype=np.int32)
    rc = _load().oracle_requant(_ptr(Y), M, N, N, _ptr(rs), _ptr(cs), float(scale), _ptr(bias_i32),
                                int(zp_out), int(bool(out_u8)), _ptr(out))
    if rc != 0:
        raise OverflowError("accumulator plus bias does not fit int32")
    return out.astype(np.uint8 if out_u8 else np.int8)


def pack_b_int8(W: np.ndarray):
    """Per-column int8 quantisation: returns (Q [K,N] int8, scale [N] f32, colsum [N] i32)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    K, N = W.shape
    Q = np.empty((K, N), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    cs = np.empty(N, dtype=np.int32)
    _load().oracle_pack_b_int8(_ptr(W), K, N, N, _ptr(Q), _ptr(s), _ptr(cs))
    return Q, s, cs


def pack_b_raw(B: np.ndarray):
    B = np.ascontiguousarray(B)
    K, N = B.shape
    Q = np.empty((K, N), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    cs = np.empty(N, dtype=np.int32)
    _load().oracle_pack_b_raw(_ptr(B), _i8kind(B), K, N, N, _ptr(Q), _ptr(s), _ptr(cs))
    return Q, s, cs


def quantize_rows_int8(X: np.ndarray):
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    Q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _load().oracle_quantize_rows_int8(_ptr(X), M, K, K, _ptr(Q), _ptr(s))
    return Q, s


def q4_1_decode(blocks: np.ndarray, K: int, N: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert blocks.size == (K // 32) * N * 20
    W = np.empty((K, N), dtype=np.float64)
    _load().oracle_q4_1_decode(_ptr(blocks), K, N, _ptr(W))
    return W


def q4_1_matmul(X: np.ndarray, blocks: np.ndarray, K: int, N: int) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float32)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    M = X.shape[0]
    assert X.shape[1] == K and blocks.size == (K // 32) * N * 20
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_q4_1_matmul(_ptr(X), M, K, K, _ptr(blocks), N, _ptr(Y), N)
    return Y


def q4_1_matmul_q8(Xq: np.ndarray, sa: np.ndarray, blocks: np.ndarray, K: int, N: int) -> np.ndarray:
    """q4_1 weights x per-row int8 activations: Xq int8 [M, K], row scales sa
    fp32 [M]; returns Y [M, N] fp64."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    M = Xq.shape[0]
    assert Xq.shape[1] == K and sa.shape == (M,) and blocks.size == (K // 32) * N * 20
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_q4_1_matmul_q8(_ptr(Xq), _ptr(sa), M, K, K, _ptr(blocks), N, _ptr(Y), N)
    return Y


def q4_1_matmul_at(X: np.ndarray, blocks: np.ndarray, K: int, N: int, im, in_) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float32)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    im = np.ascontiguousarray(im, dtype=np.int64)
    in_ = np.ascontiguousarray(in_, dtype=np.int64)
    assert (im < X.shape[0]).all() and (in_ < N).all()
    out = np.empty(im.shape, dtype=np.float64)
    _load().oracle_q4_1_matmul_at(_ptr(X), K, K, _ptr(blocks), _ptr(im), _ptr(in_), im.size, _ptr(out))
    return out


def _moe_x(X: np.ndarray, n_used: int):
    """Activations [T, K] (shared by the slots) or [T, n_used, K] (one row per
    slot): contiguous fp32 array, K, token stride and slot stride."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 2:
        return X, X.shape[1], X.shape[1], 0
    assert X.ndim == 3 and X.shape[1] == n_used
    return X, X.shape[2], X.shape[1] * X.shape[2], X.shape[2]


def q4_1_matmul_id(X: np.ndarray, experts: np.ndarray, n_expert: int, K: int, N: int,
                   ids: np.ndarray, n_used: int) -> np.ndarray:
    """X: fp32 [T, K] (shared form) or [T, n_used, K] (per-slot form); ids:
    int32 [T, ids_row_stride]; returns Y [T, n_used, N] fp64."""
    X, kx, ldx, ldx_slot = _moe_x(X, n_used)
    assert kx == K
    experts = np.ascontiguousarray(experts, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = X.shape[0]
    assert ids.shape[0] == T and ids.shape[1] >= n_used
    assert experts.size == n_expert * (K // 32) * N * 20
    Y = np.empty((T, n_used, N), dtype=np.float64)
    rc = _load().oracle_q4_1_matmul_id(_ptr(X), T, K, ldx, ldx_slot, _ptr(experts), n_expert, N, _ptr(ids),
                                        ids.shape[1], n_used, _ptr(Y), N, n_used * N)
    if rc != 0:
        raise ValueError("expert id out of range")
    return Y


def q4_1_matmul_id_at(X, experts, n_expert, K, N, ids, it, is_, in_, n_used=None) -> np.ndarray:
    """Outputs (it[i], is_[i], in_[i]); X as in q4_1_matmul_id (the per-slot
    form needs n_used)."""
    X, kx, ldx, ldx_slot = _moe_x(X, n_used if X.ndim == 3 else 0)
    assert kx == K
    experts = np.ascontiguousarray(experts, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    it = np.ascontiguousarray(it, dtype=np.int64)
    is_ = np.ascontiguousarray(is_, dtype=np.int64)
    in_ = np.ascontiguousarray(in_, dtype=np.int64)
    out = np.empty(it.shape, dtype=np.float64)
    rc = _load().oracle_q4_1_matmul_id_at(_ptr(X), K, ldx, ldx_slot, _ptr(experts), n_expert, N, _ptr(ids),
                                           ids.shape[1], _ptr(it), _ptr(is_), _ptr(in_), it.size, _ptr(out))
    if rc != 0:
        raise ValueError("expert id out of range")
    return out
