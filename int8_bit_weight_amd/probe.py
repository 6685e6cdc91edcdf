"""Binding of libqmm_probe.so, the streaming-read probe (a measurement tool
beside the product library; include/qmm_probe.h).  Argument marshalling
only; PyTorch supplies device memory and the current stream."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (binds the library to torch's HIP runtime, as the product binding does)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm_probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libqmm_probe.so is not built; run `python int8_bit_weight_amd/build.py` first")
lib = ctypes.CDLL(LIB_PATH)
lib.qmm_read_probe.restype = ctypes.c_int
lib.qmm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p]


def read_probe(buf, sink, workgroups: int, loads_per_lane: int = 4, stream=None) -> None:
    """Read every 16-byte chunk of a device buffer once; sink[w] receives the
    XOR of workgroup w's chunks."""
    s = torch.cuda.current_stream() if stream is None else stream
    st = lib.qmm_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                            ctypes.c_void_p(sink.data_ptr()), int(workgroups), int(loads_per_lane),
                            ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise RuntimeError("qmm_read_probe: status %d" % st)
