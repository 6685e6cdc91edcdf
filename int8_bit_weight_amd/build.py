"""Build libqmm.so and libqmm_probe.so (HIP, gfx950) in-tree with hipcc.

    python int8_bit_weight_amd/build.py

Every source under csrc/ is compiled for gfx950 only, with packed fp32
instructions disabled and MFMA accumulators in VGPRs, then linked into
int8_bit_weight_amd/libqmm.so (the product library, include/qmm.h).  The
streaming-read probe under probe/ becomes int8_bit_weight_amd/libqmm_probe.so
(a measurement tool, include/qmm_probe.h).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmm.so")
PROBE_SRC = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libqmm_probe.so")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with the default AGPR form the compiler
    # permuted the int8 prefill's 128 accumulators between AGPRs on every
    # k step (about 1.5 extra instructions per MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc"] + lang + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    # keep the (harmless) host-pass warning about the gfx feature out of the log
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed: %s" % lib)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    psrcs = sorted(glob.glob(os.path.join(PROBE_SRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(LIB)
        print(PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
