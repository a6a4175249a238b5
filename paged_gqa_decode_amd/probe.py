"""Binding of libtqprobe.so (include/tq_probe.h): HBM read and copy probes."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtqprobe.so")
EXPORTED_SYMBOLS = ("tq_probe_read", "tq_probe_copy")
_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_gqa_decode_amd.build`")
        lib = ctypes.CDLL(path)
        lib.tq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p]
        lib.tq_probe_read.restype = ctypes.c_int32
        lib.tq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                      ctypes.c_void_p]
        lib.tq_probe_copy.restype = ctypes.c_int32
        _lib = lib
    return _lib


def read(src: torch.Tensor, sink: torch.Tensor, num_workgroups: int, stream=None) -> None:
    assert src.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= num_workgroups
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = load_library().tq_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                      int(num_workgroups), s)
    if rc:
        raise RuntimeError(f"tq_probe_read failed: hipError {rc}")


def copy(dst: torch.Tensor, src: torch.Tensor, num_workgroups: int, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    assert dst.is_cuda and src.is_cuda and dst.numel() * dst.element_size() >= nbytes
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = load_library().tq_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, int(num_workgroups), s)
    if rc:
        raise RuntimeError(f"tq_probe_copy failed: hipError {rc}")
