"""ctypes binding of the measurement helper library libmoe_probe_mi355.so
(include/moe_probe.h): a streaming-read kernel that calibrates the HBM read
rate the weight-streaming kernels are compared against.  Argument marshalling
only."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_probe_mi355.so")
EXPORTS = ["moe_probe_stream_read"]

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        L.moe_probe_stream_read.restype = C.c_int
        L.moe_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def stream_read(buf, row_bytes: int, sink, stream=None) -> None:
    """Read the first (numel // row_bytes) * row_bytes bytes of the uint8 device
    tensor `buf` once, as rows of row_bytes (sink: a 1-element int32 device
    tensor), on `stream` (default: torch's current stream).  Returns the bytes
    read."""
    import torch
    nbytes = buf.numel() * buf.element_size() // row_bytes * row_bytes
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = lib().moe_probe_stream_read(buf.data_ptr(), nbytes, int(row_bytes), sink.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"moe_probe_stream_read failed ({rc})")
    return nbytes
