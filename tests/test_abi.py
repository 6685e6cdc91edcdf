"""CPU-only checks of the C ABI: the library loads, exports every entry point
that include/qmm.h declares, and rejects malformed arguments on the host
without touching a GPU (every case below fails validation before any HIP
call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="qmm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def q():
    import int8_bit_weight_amd as q
    return q


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["pack_b_int8", "pack_b_int8_raw", "quantize_rows_int8", "int8_gemm", "q4_1_repack",
              "q4_1_matmul", "q4_1_matmul_id", "qmm_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(q):
    for n in _declared_functions():
        assert hasattr(q.lib, n), n


def test_probe_library_is_separate(q):
    """The measurement probe lives in libqmm_probe.so (include/qmm_probe.h),
    not in the product library."""
    from int8_bit_weight_amd import probe
    assert _declared_functions("qmm_probe.h") == ["qmm_read_probe"]
    assert hasattr(probe.lib, "qmm_read_probe")
    assert not hasattr(q.lib, "qmm_read_probe")
    # rejected before any HIP call: misaligned size, bad unroll
    assert probe.lib.qmm_read_probe(FAKE, 17, FAKE, 1, 4, None) == 1
    assert probe.lib.qmm_read_probe(FAKE, 16, FAKE, 1, 3, None) == 1
    assert probe.lib.qmm_read_probe(FAKE, 0, FAKE, 1, 4, None) == 0


def test_status_strings(q):
    for s in range(5):
        assert q.lib.qmm_status_string(s)


def test_size_queries(q):
    assert q.lib.qmm_pack_b_int8_bytes(1024, 1024) == 64 + 1024 * 1024 + 8 * 1024
    assert q.lib.qmm_pack_b_int8_bytes(100, 17) == 64 + 128 * 32 + 8 * 32
    assert q.lib.qmm_int8_gemm_workspace_bytes(2048, 4096, 4096) == 0  # prefill: no split-K
    assert q.lib.qmm_int8_gemm_workspace_bytes(16, 1024, 1024) == 0  # decode: no cross-workgroup split
    # q4_1: no partial sums at M <= 4, nor at M <= 16 with K <= 1024 (one launch
    # covers the whole k range, the lm_head shape included); k splits otherwise
    assert q.lib.qmm_q4_1_matmul_workspace_bytes(4, 14336, 4096) == 0
    assert q.lib.qmm_q4_1_matmul_workspace_bytes(16, 1024, 151936) == 0
    assert q.lib.qmm_q4_1_matmul_workspace_bytes(9, 1024, 300) == 0
    assert q.lib.qmm_q4_1_matmul_workspace_bytes(16, 4096, 14336) == 4 * 16 * 14336 * 4


FAKE = ctypes.c_void_p(4096)  # never dereferenced: each call below fails validation first


def _ep(q, **kw):
    ep = q.qmm_epilogue()
    ep.outputs = kw.get("outputs", q.QMM_OUT_I32)
    ep.y_i32 = kw.get("y_i32", 4096)
    ep.ld_i32 = kw.get("ld_i32", 64)
    ep.zp_out = kw.get("zp_out", 0)
    ep.y_q8 = kw.get("y_q8", 4096)
    ep.ld_q8 = kw.get("ld_q8", 64)
    return ep


def _gemm(q, M=4, K=64, N=64, lda=64, zA=0, zB=0, at=0, bt=0, ep=None, A=FAKE, B=FAKE):
    ep = ep or _ep(q)
    return q.lib.int8_gemm(A, at, M, K, lda, zA, B, bt, N, zB, ctypes.byref(ep), None, 0, None)


def test_int8_gemm_rejections(q):
    INV, UNS = q.QMM_ERR_INVALID, q.QMM_ERR_UNSUPPORTED
    assert _gemm(q, M=-1) == INV
    assert _gemm(q, K=0) == INV
    assert _gemm(q, lda=63) == INV
    assert _gemm(q, zA=128) == INV                 # int8 A: zero point in [-128, 127]
    assert _gemm(q, at=1, zA=-1) == INV            # uint8 A: zero point in [0, 255]
    assert _gemm(q, bt=1, zB=256) == INV
    assert _gemm(q, at=2) == INV
    assert _gemm(q, ep=_ep(q, outputs=0)) == INV
    assert _gemm(q, ep=_ep(q, outputs=q.QMM_OUT_I8 | q.QMM_OUT_U8)) == INV
    assert _gemm(q, ep=_ep(q, outputs=q.QMM_OUT_I8, zp_out=128)) == INV
    assert _gemm(q, ep=_ep(q, ld_i32=63)) == INV
    assert _gemm(q, A=None) == INV
    assert _gemm(q, B=ctypes.c_void_p(4096 + 16)) == INV   # packed buffer must be 256-byte aligned
    # page bound K*255*128 < 2^31
    assert _gemm(q, K=65794, lda=65794) == UNS
    # empty products are a no-op
    assert _gemm(q, M=0) == q.QMM_OK


def test_pack_and_quantize_rejections(q):
    INV = q.QMM_ERR_INVALID
    assert q.lib.pack_b_int8(FAKE, 0, 16, 16, FAKE, 1 << 20, None) == INV
    assert q.lib.pack_b_int8(FAKE, 64, 16, 15, FAKE, 1 << 20, None) == INV
    assert q.lib.pack_b_int8(None, 64, 16, 16, FAKE, 1 << 20, None) == INV
    assert q.lib.pack_b_int8(FAKE, 64, 16, 16, ctypes.c_void_p(4096 + 64), 1 << 20, None) == INV
    assert q.lib.pack_b_int8(FAKE, 64, 16, 16, FAKE, 100, None) == q.QMM_ERR_WORKSPACE
    assert q.lib.pack_b_int8_raw(FAKE, 3, 64, 16, 16, FAKE, 1 << 20, None) == INV
    assert q.lib.quantize_rows_int8(FAKE, 4, 64, 63, FAKE, 64, FAKE, None) == INV
    assert q.lib.quantize_rows_int8(FAKE, 0, 64, 64, FAKE, 64, FAKE, None) == q.QMM_OK


def _moe(q, per_slot, T=4, K=64, ldx_slot=64, ldx=64, N=32, n_used=2, ids_stride=17, E=4, ws_bytes=1 << 24,
         ldy_slot=32, ldy_token=64, stride=None):
    stride = stride if stride is not None else q.lib.qmm_q4_1_packed_bytes(K, N) if K % 32 == 0 else 1 << 16
    stride = (stride + 255) // 256 * 256
    if per_slot:
        return q.lib.q4_1_matmul_id_per_slot(FAKE, T, K, ldx_slot, ldx, FAKE, E, N, stride, FAKE, ids_stride,
                                             n_used, FAKE, ldy_slot, ldy_token, FAKE, ws_bytes, None)
    return q.lib.q4_1_matmul_id(FAKE, T, K, ldx, FAKE, E, N, stride, FAKE, ids_stride, n_used, FAKE, ldy_slot,
                                ldy_token, FAKE, ws_bytes, None)


def test_moe_rejections(q):
    INV, UNS = q.QMM_ERR_INVALID, q.QMM_ERR_UNSUPPORTED
    assert _moe(q, False, ldx=63) == INV
    assert _moe(q, False, ids_stride=1) == INV
    assert _moe(q, False, ldy_token=63) == INV
    assert _moe(q, False, K=48, ldx=48) == UNS
    assert _moe(q, False, ws_bytes=16) == q.QMM_ERR_WORKSPACE
    assert _moe(q, False, T=0) == q.QMM_OK
    # expert counts: at least one, at most 8192 (the routing tables live in LDS)
    assert _moe(q, False, E=0) == INV
    assert _moe(q, False, n_used=0) == INV
    assert _moe(q, False, E=8193) == UNS
    # per-slot rows: ldx_slot >= K and the token stride covers n_used rows
    assert _moe(q, True, ldx_slot=63, ldx=128) == INV
    assert _moe(q, True, ldx_slot=64, ldx=127) == INV
    assert _moe(q, True, K=48, ldx_slot=48, ldx=96) == UNS
    assert _moe(q, True, ldx=128, ws_bytes=16) == q.QMM_ERR_WORKSPACE
    assert _moe(q, True, ldx=128, T=0) == q.QMM_OK
    # the per-slot workspace holds a split row per (token, slot)
    assert (q.lib.qmm_q4_1_matmul_id_per_slot_workspace_bytes(512, 8, 128, 768, 2048) >
            q.lib.qmm_q4_1_matmul_id_workspace_bytes(512, 8, 128, 768, 2048))


def test_int8_gemm_per_axis_rejections(q):
    INV = q.QMM_ERR_INVALID
    ep = _ep(q)
    f = q.lib.int8_gemm_per_axis
    assert f(FAKE, 0, 4, 64, 64, ctypes.c_void_p(4098), FAKE, 0, 64, None, ctypes.byref(ep), None, 0, None) == INV
    assert f(FAKE, 0, 4, 64, 64, None, FAKE, 0, 64, ctypes.c_void_p(4098), ctypes.byref(ep), None, 0, None) == INV
    assert f(FAKE, 0, 4, 64, 63, None, FAKE, 0, 64, None, ctypes.byref(ep), None, 0, None) == INV
    assert f(FAKE, 2, 4, 64, 64, None, FAKE, 0, 64, None, ctypes.byref(ep), None, 0, None) == INV
    assert f(FAKE, 0, 0, 64, 64, FAKE, FAKE, 0, 64, FAKE, ctypes.byref(ep), None, 0, None) == q.QMM_OK


def test_q4_1_matmul_q8_rejections(q):
    INV, UNS = q.QMM_ERR_INVALID, q.QMM_ERR_UNSUPPORTED
    f = q.lib.q4_1_matmul_q8
    assert f(FAKE, FAKE, 4, 64, 63, FAKE, 16, FAKE, 16, None) == INV       # ldq < K
    assert f(FAKE, FAKE, 4, 64, 64, FAKE, 16, FAKE, 15, None) == INV       # ldy < N
    assert f(FAKE, FAKE, 4, 48, 48, FAKE, 16, FAKE, 16, None) == UNS       # K % 32
    assert f(FAKE, None, 4, 64, 64, FAKE, 16, FAKE, 16, None) == INV       # no row scales
    assert f(FAKE, FAKE, 4, 64, 64, ctypes.c_void_p(4096 + 16), 16, FAKE, 16, None) == INV
    assert f(FAKE, FAKE, 0, 64, 64, FAKE, 16, FAKE, 16, None) == q.QMM_OK


def test_check_mode_toggle(q):
    q.lib.qmm_set_check(1)
    assert q.lib.qmm_check_enabled() == 1
    q.lib.qmm_set_check(0)
    assert q.lib.qmm_check_enabled() == 0


def test_moe_noalloc_rejections(q):
    """The allocation-free MUL_MAT_ID checks its arguments like the workspace
    form and refuses, before any HIP call, a problem whose scratch would not
    fit the library's array."""
    INV, WS = q.QMM_ERR_INVALID, q.QMM_ERR_WORKSPACE
    f = q.lib.q4_1_matmul_id_noalloc
    stride = (q.lib.qmm_q4_1_packed_bytes(4096, 768) + 255) // 256 * 256
    assert q.lib.qmm_q4_1_matmul_id_workspace_bytes(512, 8, 128, 2048, 768) <= 16 << 20
    need = q.lib.qmm_q4_1_matmul_id_workspace_bytes(8192, 8, 128, 4096, 768)
    assert need > 16 << 20
    assert f(FAKE, 8192, 4096, 4096, FAKE, 128, 768, stride, FAKE, 17, 8, FAKE, 768, 8 * 768, None) == WS
    assert f(FAKE, 4, 64, 63, FAKE, 4, 32, 1 << 16, FAKE, 17, 2, FAKE, 32, 64, None) == INV     # ldx < K
    assert f(None, 4, 64, 64, FAKE, 4, 32, 1 << 16, FAKE, 17, 2, FAKE, 32, 64, None) == INV      # no X
    assert f(FAKE, 0, 64, 64, FAKE, 4, 32, 1 << 16, FAKE, 17, 2, FAKE, 32, 64, None) == q.QMM_OK


def test_dynamic_grouped_rejections(q):
    """The grouped dynamic call checks every item before anything runs."""
    INV = q.QMM_ERR_INVALID
    f = q.lib.int8_gemm_dynamic_grouped

    def items(*spec):
        arr = (q.qmm_dynamic_item * len(spec))()
        for i, (pk, n, y, ld) in enumerate(spec):
            arr[i].packedB, arr[i].N, arr[i].y_f32, arr[i].ld_f32, arr[i].bias_f32 = pk, n, y, ld, None
        return arr
    ok = items((4096, 64, 4096, 64), (4096, 32, 4096, 32))
    assert f(FAKE, 4, 64, 63, ok, 2, 1.0, None, 0, None) == INV                    # ldx < K
    assert f(FAKE, 4, 64, 64, ok, 0, 1.0, None, 0, None) == INV                    # no items
    assert f(FAKE, 4, 64, 64, items(*[(4096, 16, 4096, 16)] * 5), 5, 1.0, None, 0, None) == INV  # > 4 items
    assert f(FAKE, 4, 64, 64, items((4096, 64, 4096, 63)), 1, 1.0, None, 0, None) == INV     # ld < N
    assert f(FAKE, 4, 64, 64, items((4096 + 16, 64, 4096, 64)), 1, 1.0, None, 0, None) == INV  # alignment
    assert f(FAKE, 4, 64, 64, items((4096, 64, None, 64)), 1, 1.0, None, 0, None) == INV     # no output
    assert f(None, 4, 64, 64, ok, 2, 1.0, None, 0, None) == INV
    assert f(FAKE, 0, 64, 64, ok, 2, 1.0, None, 0, None) == q.QMM_OK
    assert f(FAKE, 4, 65794, 65794, ok, 2, 1.0, None, 0, None) == q.QMM_ERR_UNSUPPORTED   # the K bound
    assert q.lib.qmm_int8_gemm_dynamic_grouped_workspace_bytes(16, 1024) == 0
    assert q.lib.qmm_int8_gemm_dynamic_grouped_workspace_bytes(40, 1024) == 0    # eight row groups
    assert q.lib.qmm_int8_gemm_dynamic_grouped_workspace_bytes(200, 256) > 0
    assert q.lib.qmm_int8_gemm_dynamic_grouped_workspace_bytes(4, 5120) > 0
