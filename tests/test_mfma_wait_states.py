"""CPU check of the built kernels: no control-flow path reads an MFMA result
with fewer wait states than the compiler leaves for the same MFMA on
straight-line code.

A wave-uniform branch that skipped a row tile's MFMAs once let the branch-taken
path read an accumulator one instruction after its MFMA (the fall-through path
carried the s_nop), so chunks of <= 16 rows summed stale registers.  This test
compiles every kernel source of the library to gfx950 assembly with the build
flags and walks every path (tests/mfma_paths.py).
"""
import concurrent.futures as cf
import glob
import importlib.util
import os
import shutil
import subprocess
import tempfile

import pytest

from mfma_paths import functions, raw_distances

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_bit_weight_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")


def _build_flags():
    spec = importlib.util.spec_from_file_location("_qmm_build", os.path.join(ROOT, "int8_bit_weight_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.CFLAGS


@pytest.fixture(scope="module")
def assembly():
    flags = _build_flags()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = tempfile.mkdtemp(prefix="qmm_asm_")

    def one(src):
        out = os.path.join(tmp, os.path.basename(src) + ".s")
        r = subprocess.run(["hipcc", "-x", "hip"] + flags + ["--cuda-device-only", "-S", src, "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return os.path.basename(src), f.read()

    try:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            yield dict(ex.map(one, srcs))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_path_keeps_the_mfma_result_wait(assembly):
    rows = []
    for name, asm in assembly.items():
        for func, body in functions(asm):
            for op, w_any, w_ft, reader in raw_distances(body):
                rows.append((name, func, op, w_any, w_ft, reader))
    assert rows, "no MFMA result readers found: the assembly was not parsed"
    # the compiler's own requirement per MFMA opcode: the fewest wait states
    # it leaves on a fall-through path anywhere in the library
    need = {}
    for _, _, op, _, w_ft, _ in rows:
        if w_ft < 99:
            need[op] = min(need.get(op, 99), w_ft)
    bad = [r for r in rows if r[3] < need.get(r[2], 0)]
    assert not bad, "\n".join("%s %s: %s read %d wait states after %s (straight-line code keeps %d)"
                              % (n, f[:60], rd, w, op, need[op]) for n, f, op, w, _, rd in bad[:20])


def test_scanner_sees_a_skipped_wait():
    """The scanner itself: a branch over the padding is reported."""
    body = """
	v_mfma_f32_16x16x32_f16 v[4:7], v[0:3], v[8:11], 0
	s_cbranch_vccnz .LBB0_2
; %bb.1:
	s_nop 7
	v_add_f32_e32 v12, v4, v4
.LBB0_2:
	v_add_f32_e32 v13, v5, v5
	s_endpgm
""".split("\n")
    got = {(rd.split()[0], w_any, w_ft) for _, w_any, w_ft, rd in raw_distances(body)}
    # v12 is read 9 wait states after the MFMA (branch + s_nop 7); v13 one
    # after it on the taken path, 10 on the fall-through path
    assert ("v_add_f32_e32", 9, 9) in got
    assert ("v_add_f32_e32", 1, 10) in got
