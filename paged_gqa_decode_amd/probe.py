"""Binding of libtqprobe.so (include/tq_probe.h): HBM read, copy and decode-pattern probes."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtqprobe.so")
EXPORTED_SYMBOLS = ("tq_probe_read", "tq_probe_copy", "tq_probe_pattern", "tq_probe_pattern4")
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
        lib.tq_probe_pattern.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.tq_probe_pattern.restype = ctypes.c_int32
        lib.tq_probe_pattern4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
        lib.tq_probe_pattern4.restype = ctypes.c_int32
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


def pattern(k: torch.Tensor, v: torch.Tensor, scales: torch.Tensor, chunks_per_wave: int,
            num_workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """The decode's byte pattern with no arithmetic (tq_probe_pattern)."""
    assert k.is_cuda and v.is_cuda and scales.is_cuda and sink.is_cuda and sink.numel() >= num_workgroups
    kvb = min(k.numel() * k.element_size(), v.numel() * v.element_size())
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = load_library().tq_probe_pattern(k.data_ptr(), v.data_ptr(), scales.data_ptr(), kvb,
                                         scales.numel() * scales.element_size(), int(chunks_per_wave),
                                         int(num_workgroups), sink.data_ptr(), s)
    if rc:
        raise RuntimeError(f"tq_probe_pattern failed: hipError {rc}")


def pattern4(rows: torch.Tensor, meta: torch.Tensor, chunks_per_wave: int, num_workgroups: int,
             sink: torch.Tensor, stream=None) -> None:
    """The 4-bit format's byte pattern with no arithmetic (tq_probe_pattern4)."""
    assert rows.is_cuda and meta.is_cuda and sink.is_cuda and sink.numel() >= num_workgroups
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = load_library().tq_probe_pattern4(rows.data_ptr(), meta.data_ptr(),
                                          rows.numel() * rows.element_size(),
                                          meta.numel() * meta.element_size(), int(chunks_per_wave),
                                          int(num_workgroups), sink.data_ptr(), s)
    if rc:
        raise RuntimeError(f"tq_probe_pattern4 failed: hipError {rc}")
