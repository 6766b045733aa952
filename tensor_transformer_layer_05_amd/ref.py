"""Binding of libtpref.so, the measurement reference kernels (not part of the
layer): ``stream_read`` reads a device buffer once with the decode
weight-streaming kernels' access shape, to measure the attainable HBM read
rate next to them.  Argument marshalling only; raises if the library is
missing."""
from __future__ import annotations

import ctypes
import os

import torch

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpref.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run __graft_entry__.build()")
        l = ctypes.CDLL(library_path)
        l.tpref_stream_read.restype = ctypes.c_int
        l.tpref_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _lib = l
    return _lib


# flags of stream_read
NONTEMPORAL = 1   # streaming cache policy on every load
SPREAD = 2        # chunks interleaved over all waves instead of a slice per wave


def stream_read(buf: torch.Tensor, out: torch.Tensor, workgroups: int = 256, waves: int = 8,
                loads_per_lane: int = 8, flags: int = 0) -> torch.Tensor:
    """Read all of ``buf`` (a contiguous device tensor) once; ``out`` is a
    uint32-sized device tensor of at least ``workgroups * waves * 64``
    elements receiving one folded word per lane; ``flags`` a combination of
    NONTEMPORAL and SPREAD."""
    if not (buf.is_cuda and out.is_cuda and buf.is_contiguous() and out.is_contiguous()):
        raise ValueError("buf and out must be contiguous device tensors")
    if out.numel() * out.element_size() < workgroups * waves * 64 * 4:
        raise ValueError("out too small")
    st = lib().tpref_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                 workgroups, waves, loads_per_lane, flags,
                                 ctypes.c_void_p(torch.cuda.current_stream(buf.device).cuda_stream))
    if st != 0:
        raise RuntimeError(f"tpref_stream_read failed with status {st}")
    return out
