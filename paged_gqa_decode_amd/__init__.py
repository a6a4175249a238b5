"""Python binding of libtqdecode.so: paged grouped-query decode attention over an
fp8 e4m3fn paged KV cache on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/tq_decode.h.  torch provides the
device memory and the current stream.  If the built library is missing, or
the arguments are not tensors on a GPU, the calls raise -- there is no other
implementation to fall back to.

Names follow the C ABI: ``tq_decode`` (partition kernel, writes the split-K
partial triple), ``tq_decode_reduce`` (log-sum-exp merge into bf16), plus
``decode`` (both, with the partials and output allocated here).
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtqdecode.so")

HEAD_DIM = 128
TOKENS_PER_TILE_GROUP = 256
SUPPORTED_QUERY_GROUP_SIZES = (6, 8, 16)
SUPPORTED_KV_BLOCK_SIZES = (16, 32)

TQ_OK, TQ_ERR_NULL, TQ_ERR_MISALIGNED, TQ_ERR_UNSUPPORTED, TQ_ERR_SHAPE, TQ_ERR_COVERAGE, \
    TQ_ERR_SCALE, TQ_ERR_HIP, TQ_ERR_SCRATCH = range(9)
STATIC_SCRATCH_BYTES = 8 << 20
STATIC_COUNTER_BYTES = 1 << 20

EXPORTED_SYMBOLS = ("tq_decode", "tq_decode_reduce", "tq_decode_fused", "tq_decode_fused_static",
                    "tq_fused_workspace_bytes",
                    "tq4_decode", "tq4_decode_fused", "tq4_block_bytes", "tq_kv_write",
                    "tq_partials_bytes", "tq_status_str", "tq_last_hip_error", "tq_abi_version")


class TqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_str(status)})")
        self.status = status


# Order of the 128-byte K / V rows inside a cache block: "head" [Hkv][BS] (the default, the
# faster stream) or "slot" [BS][Hkv] (the page's data region).
KV_LAYOUTS = {"head": 0, "slot": 1}


class Extent(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_layout", ctypes.c_int32)]


class PartialsStruct(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("max_logits", ctypes.c_void_p),
                ("exp_sums", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_gqa_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.tq_decode.argtypes = [P, P, P, P, P, P, ctypes.POINTER(PartialsStruct), i32, i32, i32, i32,
                              ctypes.c_float, ctypes.POINTER(Extent), P]
    lib.tq_decode.restype = ctypes.c_int
    lib.tq_decode_reduce.argtypes = [ctypes.POINTER(PartialsStruct), P, P, i32, i32, i32,
                                     ctypes.POINTER(Extent), P]
    lib.tq_decode_reduce.restype = ctypes.c_int
    lib.tq_decode_fused.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float,
                                    ctypes.POINTER(Extent), P, ctypes.c_size_t, P]
    lib.tq_decode_fused.restype = ctypes.c_int
    lib.tq_decode_fused_static.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float,
                                           ctypes.POINTER(Extent), P]
    lib.tq_decode_fused_static.restype = ctypes.c_int
    lib.tq4_decode.argtypes = [P, P, P, P, P, ctypes.POINTER(PartialsStruct), i32, i32, i32, i32,
                               ctypes.c_float, ctypes.POINTER(Extent), P]
    lib.tq4_decode.restype = ctypes.c_int
    lib.tq4_decode_fused.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float,
                                     ctypes.POINTER(Extent), P, ctypes.c_size_t, P]
    lib.tq4_decode_fused.restype = ctypes.c_int
    lib.tq4_block_bytes.argtypes = [i32, i32]
    lib.tq4_block_bytes.restype = ctypes.c_size_t
    lib.tq_kv_write.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, P]
    lib.tq_kv_write.restype = ctypes.c_int
    lib.tq_fused_workspace_bytes.argtypes = [ctypes.POINTER(Extent), i32, i32]
    lib.tq_fused_workspace_bytes.restype = ctypes.c_size_t
    lib.tq_partials_bytes.argtypes = [ctypes.POINTER(Extent), i32, i32]
    lib.tq_partials_bytes.restype = ctypes.c_size_t
    lib.tq_status_str.argtypes = [ctypes.c_int]
    lib.tq_status_str.restype = ctypes.c_char_p
    lib.tq_last_hip_error.argtypes = []
    lib.tq_last_hip_error.restype = ctypes.c_int32
    lib.tq_abi_version.argtypes = []
    lib.tq_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().tq_status_str(int(status)).decode()


def abi_version() -> int:
    return int(load_library().tq_abi_version())


def last_hip_error() -> int:
    return int(load_library().tq_last_hip_error())


@dataclass
class Partials:
    """The split-K partial triple: out [S][Hkv][P][QG][128], max_logits / exp_sums [S][Hkv][P][QG] (fp32)."""
    out: torch.Tensor
    max_logits: torch.Tensor
    exp_sums: torch.Tensor

    def _struct(self) -> PartialsStruct:
        return PartialsStruct(self.out.data_ptr(), self.max_logits.data_ptr(), self.exp_sums.data_ptr())


def alloc_partials(num_seqs: int, num_kv_heads: int, num_partitions: int, query_group_size: int,
                   device) -> Partials:
    shape = (num_seqs, num_kv_heads, num_partitions, query_group_size)
    return Partials(out=torch.empty(shape + (HEAD_DIM,), dtype=torch.float32, device=device),
                    max_logits=torch.empty(shape, dtype=torch.float32, device=device),
                    exp_sums=torch.empty(shape, dtype=torch.float32, device=device))


def _layout(kv_layout: str) -> int:
    if kv_layout not in KV_LAYOUTS:
        raise ValueError(f"kv_layout must be one of {sorted(KV_LAYOUTS)}, not {kv_layout!r}")
    return KV_LAYOUTS[kv_layout]


def _extent(num_seqs, num_blocks, max_blocks_per_seq, num_partitions, max_seq_len,
            kv_layout: str = "head") -> Extent:
    return Extent(int(num_seqs), int(num_blocks), int(max_blocks_per_seq), int(num_partitions),
                  int(max_seq_len), HEAD_DIM, _layout(kv_layout))


def cache_shape(num_blocks: int, num_kv_heads: int, kv_block_size: int, kv_layout: str = "head"):
    """Shape of an fp8 k_cache / v_cache in the given row order."""
    _layout(kv_layout)
    return ((num_blocks, num_kv_heads, kv_block_size, HEAD_DIM) if kv_layout == "head"
            else (num_blocks, kv_block_size, num_kv_heads, HEAD_DIM))


def partials_bytes(num_seqs, num_kv_heads, num_partitions, query_group_size) -> int:
    ext = _extent(num_seqs, 1, 1, num_partitions, 0)
    return int(load_library().tq_partials_bytes(ctypes.byref(ext), int(num_kv_heads),
                                                int(query_group_size)))


_FP8_CODES = (torch.uint8, torch.float8_e4m3fn)


def _expect(t, name: str, dtypes, shape) -> None:
    """Refuse a tensor whose dtype or shape disagrees with what the entry point will read or
    write through its pointer (None in `shape` matches any size).  Checked before the device,
    so that a wrong layout never reaches a kernel."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if t.dim() != len(shape) or any(w is not None and int(n) != int(w) for n, w in zip(t.shape, shape)):
        want = tuple("*" if w is None else int(w) for w in shape)
        raise ValueError(f"{name} must have shape {want}, not {tuple(t.shape)}")


def _expect_partials(partials: "Partials", S: int, Hkv: int, P: int, QG: int) -> None:
    _expect(partials.out, "partials.out", torch.float32, (S, Hkv, P, QG, HEAD_DIM))
    _expect(partials.max_logits, "partials.max_logits", torch.float32, (S, Hkv, P, QG))
    _expect(partials.exp_sums, "partials.exp_sums", torch.float32, (S, Hkv, P, QG))


def _expect_pool(num_blocks: int, *tensors) -> None:
    for t, name in tensors:
        if num_blocks > int(t.shape[0]):
            raise ValueError(f"num_blocks {num_blocks} exceeds the {int(t.shape[0])} blocks of {name}")


def _expect_fp8_inputs(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, Hkv, QG, BS,
                       kv_layout="head"):
    """q, the fp8 cache pair with its scales, the block table and the lengths; returns S."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [S][Hkv*QG][128] tensor")
    S = int(q.shape[0])
    _expect(q, "q", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    shape = (None,) + cache_shape(1, Hkv, BS, kv_layout)[1:]
    _expect(k_cache, "k_cache", _FP8_CODES, shape)
    _expect(v_cache, "v_cache", _FP8_CODES, shape)
    _expect(kv_scales, "kv_scales", torch.float32, (None, Hkv, 2, BS))
    _expect(block_tables, "block_tables", torch.int32, (S, None))
    _expect(seq_lens, "seq_lens", torch.int32, (S,))
    return S


def _expect_tq4_inputs(lib, q_rot, kv_cache, centroids, block_tables, seq_lens, Hkv, QG, BS):
    """q, the 4-bit record pool, the centroids, the block table and the lengths; returns S."""
    if not isinstance(q_rot, torch.Tensor) or q_rot.dim() != 3:
        raise ValueError("q_rot must be a [S][Hkv*QG][128] tensor")
    S = int(q_rot.shape[0])
    _expect(q_rot, "q_rot", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    bb = int(lib.tq4_block_bytes(int(Hkv), int(BS)))
    _expect(kv_cache, "kv_cache", torch.uint8, (None, bb if bb > 0 else None))
    _expect(centroids, "centroids", torch.float32, (16,))
    _expect(block_tables, "block_tables", torch.int32, (S, None))
    _expect(seq_lens, "seq_lens", torch.int32, (S,))
    return S


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_stream(stream):
    """Context in which `stream` (a torch stream, a raw hipStream_t handle, or None for the
    current stream) is torch's current stream: temporaries allocated inside it belong to that
    stream in torch's caching allocator, so that they are ordered with the kernels enqueued
    there and are not handed out again while those kernels may still use them."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(_stream(stream))
    return torch.cuda.stream(stream)


def tq_decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, partials: Partials,
              num_kv_heads: int, query_group_size: int, kv_block_size: int,
              tile_groups_per_partition: int, softmax_scale: float, *, num_partitions: int,
              max_seq_len: int, num_blocks: Optional[int] = None, kv_layout: str = "head",
              stream=None) -> None:
    """Enqueue the partition kernel (C ABI tq_decode); writes `partials` for live partitions."""
    lib = load_library()
    Hkv, QG, BS = int(num_kv_heads), int(query_group_size), int(kv_block_size)
    S = _expect_fp8_inputs(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, Hkv, QG, BS,
                           kv_layout)
    _expect_partials(partials, S, Hkv, int(num_partitions), QG)
    nb = int(k_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _expect_pool(nb, (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_scales, "kv_scales"))
    ptrs = [_dev(t, n) for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                                    (kv_scales, "kv_scales"), (block_tables, "block_tables"),
                                    (seq_lens, "seq_lens"))]
    for t, n in ((partials.out, "partials.out"), (partials.max_logits, "partials.max_logits"),
                 (partials.exp_sums, "partials.exp_sums")):
        _dev(t, n)
    ext = _extent(q.shape[0], nb, block_tables.shape[1], num_partitions, max_seq_len, kv_layout)
    ps = partials._struct()
    st = lib.tq_decode(*ptrs, ctypes.byref(ps), int(num_kv_heads), int(query_group_size),
                       int(kv_block_size), int(tile_groups_per_partition), float(softmax_scale),
                       ctypes.byref(ext), _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq_decode")


def tq_decode_reduce(partials: Partials, seq_lens, out, num_kv_heads: int, query_group_size: int,
                     tile_groups_per_partition: int, *, num_partitions: int, max_seq_len: int,
                     stream=None) -> None:
    """Enqueue the merge kernel (C ABI tq_decode_reduce) into bf16 `out` [S][Hkv*QG][128]."""
    lib = load_library()
    if not isinstance(out, torch.Tensor) or out.dim() != 3:
        raise ValueError("out must be a [S][Hkv*QG][128] tensor")
    S, Hkv, QG = int(out.shape[0]), int(num_kv_heads), int(query_group_size)
    _expect(out, "out", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    _expect(seq_lens, "seq_lens", torch.int32, (S,))
    _expect_partials(partials, S, Hkv, int(num_partitions), QG)
    for t, n in ((partials.out, "partials.out"), (partials.max_logits, "partials.max_logits"),
                 (partials.exp_sums, "partials.exp_sums")):
        _dev(t, n)
    ext = _extent(out.shape[0], 1, 1, num_partitions, max_seq_len)
    ps = partials._struct()
    st = lib.tq_decode_reduce(ctypes.byref(ps), _dev(seq_lens, "seq_lens"), _dev(out, "out"),
                              int(num_kv_heads), int(query_group_size),
                              int(tile_groups_per_partition), ctypes.byref(ext), _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq_decode_reduce")


def fused_workspace_bytes(num_seqs, num_kv_heads, query_group_size, max_seq_len) -> int:
    ext = _extent(num_seqs, 1, 1, 1, max_seq_len)
    return int(load_library().tq_fused_workspace_bytes(ctypes.byref(ext), int(num_kv_heads),
                                                       int(query_group_size)))


def alloc_fused_workspace(num_seqs, num_kv_heads, query_group_size, max_seq_len,
                          device) -> Optional[torch.Tensor]:
    """Zero-filled workspace for tq_decode_fused (None when it needs none)."""
    n = fused_workspace_bytes(num_seqs, num_kv_heads, query_group_size, max_seq_len)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def tq_decode_fused(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, out,
                    num_kv_heads: int, query_group_size: int, kv_block_size: int,
                    tile_groups_per_partition: int, softmax_scale: float, *, num_partitions: int,
                    max_seq_len: int, num_blocks: Optional[int] = None,
                    workspace: Optional[torch.Tensor] = None, kv_layout: str = "head",
                    stream=None) -> None:
    """Enqueue the one-launch decode (C ABI tq_decode_fused) into bf16 `out` [S][Hkv*QG][128].
    `workspace`: None or a zero-filled uint8 device tensor (see alloc_fused_workspace)."""
    lib = load_library()
    Hkv, QG, BS = int(num_kv_heads), int(query_group_size), int(kv_block_size)
    S = _expect_fp8_inputs(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, Hkv, QG, BS,
                           kv_layout)
    _expect(out, "out", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    nb = int(k_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _expect_pool(nb, (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_scales, "kv_scales"))
    ptrs = [_dev(t, n) for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                                    (kv_scales, "kv_scales"), (block_tables, "block_tables"),
                                    (seq_lens, "seq_lens"), (out, "out"))]
    ext = _extent(q.shape[0], nb, block_tables.shape[1], num_partitions, max_seq_len, kv_layout)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.tq_decode_fused(*ptrs, int(num_kv_heads), int(query_group_size), int(kv_block_size),
                             int(tile_groups_per_partition), float(softmax_scale),
                             ctypes.byref(ext), ws_ptr, ws_bytes, _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq_decode_fused")


def tq_decode_fused_static(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, out,
                           num_kv_heads: int, query_group_size: int, kv_block_size: int,
                           tile_groups_per_partition: int, softmax_scale: float, *,
                           num_partitions: int, max_seq_len: int, num_blocks: Optional[int] = None,
                           kv_layout: str = "head", stream=None) -> None:
    """Enqueue the one-launch decode with the library's static scratch (C ABI
    tq_decode_fused_static): nothing is allocated, here or in the library."""
    lib = load_library()
    Hkv, QG, BS = int(num_kv_heads), int(query_group_size), int(kv_block_size)
    S = _expect_fp8_inputs(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, Hkv, QG, BS,
                           kv_layout)
    _expect(out, "out", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    nb = int(k_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _expect_pool(nb, (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_scales, "kv_scales"))
    ptrs = [_dev(t, n) for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                                    (kv_scales, "kv_scales"), (block_tables, "block_tables"),
                                    (seq_lens, "seq_lens"), (out, "out"))]
    ext = _extent(q.shape[0], nb, block_tables.shape[1], num_partitions, max_seq_len, kv_layout)
    st = lib.tq_decode_fused_static(*ptrs, Hkv, QG, BS, int(tile_groups_per_partition),
                                    float(softmax_scale), ctypes.byref(ext), _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq_decode_fused_static")


def tq4_block_bytes(num_kv_heads: int, kv_block_size: int) -> int:
    """Bytes of one cache block of the 4-bit record format (C ABI tq4_block_bytes)."""
    return int(load_library().tq4_block_bytes(int(num_kv_heads), int(kv_block_size)))


def tq4_decode(q_rot, kv_cache, centroids, block_tables, seq_lens, partials: Partials,
               num_kv_heads: int, query_group_size: int, kv_block_size: int,
               tile_groups_per_partition: int, softmax_scale: float, *, num_partitions: int,
               max_seq_len: int, num_blocks: Optional[int] = None, kv_layout: str = "head",
              stream=None) -> None:
    """Enqueue the partition kernel over the 4-bit record format (C ABI tq4_decode)."""
    lib = load_library()
    Hkv, QG, BS = int(num_kv_heads), int(query_group_size), int(kv_block_size)
    S = _expect_tq4_inputs(lib, q_rot, kv_cache, centroids, block_tables, seq_lens, Hkv, QG, BS)
    _expect_partials(partials, S, Hkv, int(num_partitions), QG)
    nb = int(kv_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _expect_pool(nb, (kv_cache, "kv_cache"))
    ptrs = [_dev(t, n) for t, n in ((q_rot, "q_rot"), (kv_cache, "kv_cache"),
                                    (centroids, "centroids"), (block_tables, "block_tables"),
                                    (seq_lens, "seq_lens"))]
    for t, n in ((partials.out, "partials.out"), (partials.max_logits, "partials.max_logits"),
                 (partials.exp_sums, "partials.exp_sums")):
        _dev(t, n)
    ext = _extent(q_rot.shape[0], nb, block_tables.shape[1], num_partitions, max_seq_len,
                  kv_layout)
    ps = partials._struct()
    st = lib.tq4_decode(*ptrs, ctypes.byref(ps), int(num_kv_heads), int(query_group_size),
                        int(kv_block_size), int(tile_groups_per_partition), float(softmax_scale),
                        ctypes.byref(ext), _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq4_decode")


def tq4_decode_fused(q_rot, kv_cache, centroids, block_tables, seq_lens, out, num_kv_heads: int,
                     query_group_size: int, kv_block_size: int, tile_groups_per_partition: int,
                     softmax_scale: float, *, num_partitions: int, max_seq_len: int,
                     num_blocks: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                     kv_layout: str = "head", stream=None) -> None:
    """Enqueue the one-launch decode over the 4-bit record format (C ABI tq4_decode_fused)."""
    lib = load_library()
    Hkv, QG, BS = int(num_kv_heads), int(query_group_size), int(kv_block_size)
    S = _expect_tq4_inputs(lib, q_rot, kv_cache, centroids, block_tables, seq_lens, Hkv, QG, BS)
    _expect(out, "out", torch.bfloat16, (S, Hkv * QG, HEAD_DIM))
    nb = int(kv_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _expect_pool(nb, (kv_cache, "kv_cache"))
    ptrs = [_dev(t, n) for t, n in ((q_rot, "q_rot"), (kv_cache, "kv_cache"),
                                    (centroids, "centroids"), (block_tables, "block_tables"),
                                    (seq_lens, "seq_lens"), (out, "out"))]
    ext = _extent(q_rot.shape[0], nb, block_tables.shape[1], num_partitions, max_seq_len,
                  kv_layout)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.tq4_decode_fused(*ptrs, int(num_kv_heads), int(query_group_size), int(kv_block_size),
                              int(tile_groups_per_partition), float(softmax_scale),
                              ctypes.byref(ext), ws_ptr, ws_bytes, _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq4_decode_fused")


def decode_tq4(q_rot, kv_cache, centroids, block_tables, seq_lens, *, num_kv_heads: int,
               kv_block_size: int, num_partitions=None, tile_groups_per_partition: int = 1,
               softmax_scale: Optional[float] = None, max_seq_len: Optional[int] = None,
               partials: Optional[Partials] = None, out: Optional[torch.Tensor] = None,
               fused: bool = False, workspace: Optional[torch.Tensor] = None,
               kv_layout: str = "head", stream=None) -> torch.Tensor:
    """decode() for the 4-bit record format: kv_cache uint8 [NB][tq4_block_bytes] (data rows
    in the order `kv_layout` names), centroids fp32 [16], q_rot bf16 [S][Hq][128].  Returns
    bf16 [S][Hq][128]."""
    with _on_stream(stream):
        return _decode_tq4(q_rot, kv_cache, centroids, block_tables, seq_lens, num_kv_heads,
                           kv_block_size, num_partitions, tile_groups_per_partition,
                           softmax_scale, max_seq_len, partials, out, fused, workspace, kv_layout,
                           stream)


def _decode_tq4(q_rot, kv_cache, centroids, block_tables, seq_lens, num_kv_heads, kv_block_size,
                num_partitions, tile_groups_per_partition, softmax_scale, max_seq_len, partials,
                out, fused, workspace, kv_layout, stream):
    S, Hq, D = q_rot.shape
    Hkv, BS = int(num_kv_heads), int(kv_block_size)
    if D != HEAD_DIM or Hq % Hkv:
        raise ValueError("head_dim must be 128 and num_q_heads a multiple of num_kv_heads")
    QG = Hq // Hkv
    G = int(tile_groups_per_partition)
    if max_seq_len is None:
        if torch.cuda.is_current_stream_capturing():
            max_seq_len = int(block_tables.shape[1]) * BS
        else:
            max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    if num_partitions is None:
        num_partitions = max(1, -(-int(max_seq_len) // (TOKENS_PER_TILE_GROUP * G)))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((S, Hq, HEAD_DIM), dtype=torch.bfloat16, device=q_rot.device)
    if fused:
        if workspace is None:
            workspace = alloc_fused_workspace(S, Hkv, QG, max_seq_len, q_rot.device)
        tq4_decode_fused(q_rot, kv_cache, centroids, block_tables, seq_lens, out, Hkv, QG, BS, G,
                         softmax_scale, num_partitions=num_partitions, max_seq_len=max_seq_len,
                         workspace=workspace, kv_layout=kv_layout, stream=stream)
        return out
    if partials is None:
        partials = alloc_partials(S, Hkv, num_partitions, QG, q_rot.device)
    tq4_decode(q_rot, kv_cache, centroids, block_tables, seq_lens, partials, Hkv, QG, BS, G,
               softmax_scale, num_partitions=num_partitions, max_seq_len=max_seq_len,
               kv_layout=kv_layout, stream=stream)
    tq_decode_reduce(partials, seq_lens, out, Hkv, QG, G, num_partitions=num_partitions,
                     max_seq_len=max_seq_len, stream=stream)
    return out


def tq_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache, kv_scales, *,
                kv_layout: str = "head", stream=None) -> None:
    """Enqueue the KV-cache writer (C ABI tq_kv_write): quantize the new bf16 K/V rows
    [T][Hkv][128] and store them at slot_mapping (int32 [T], negative = skip) in a cache of
    the given row order ([NB][Hkv][BS][128] "head" or [NB][BS][Hkv][128] "slot")."""
    lib = load_library()
    if not isinstance(k_new, torch.Tensor) or k_new.dim() != 3 or not isinstance(k_cache, torch.Tensor) \
            or k_cache.dim() != 4:
        raise ValueError("k_new must be [T][Hkv][128] and k_cache a 4-d cache tensor")
    T, Hkv, D = (int(n) for n in k_new.shape)
    NB = int(k_cache.shape[0])
    BS = int(k_cache.shape[2] if kv_layout == "head" else k_cache.shape[1])
    _expect(k_new, "k_new", torch.bfloat16, (T, Hkv, HEAD_DIM))
    _expect(v_new, "v_new", torch.bfloat16, (T, Hkv, HEAD_DIM))
    _expect(slot_mapping, "slot_mapping", torch.int32, (T,))
    _expect(k_cache, "k_cache", _FP8_CODES, cache_shape(NB, Hkv, BS, kv_layout))
    _expect(v_cache, "v_cache", _FP8_CODES, cache_shape(NB, Hkv, BS, kv_layout))
    _expect(kv_scales, "kv_scales", torch.float32, (NB, Hkv, 2, BS))
    if T == 0:
        return
    ptrs = [_dev(t, n) for t, n in ((k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"),
                                    (k_cache, "k_cache"), (v_cache, "v_cache"),
                                    (kv_scales, "kv_scales"))]
    st = lib.tq_kv_write(*ptrs, int(T), int(Hkv), int(BS), int(NB), int(D), _layout(kv_layout),
                         _stream(stream))
    if st != TQ_OK:
        raise TqError(st, "tq_kv_write")


def decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, *, num_partitions=None,
           tile_groups_per_partition: int = 1, softmax_scale: Optional[float] = None,
           max_seq_len: Optional[int] = None, partials: Optional[Partials] = None,
           out: Optional[torch.Tensor] = None, fused: bool = False,
           workspace: Optional[torch.Tensor] = None, kv_layout: str = "head",
           stream=None) -> torch.Tensor:
    """Decode attention; returns bf16 [S][Hkv*QG][128].

    fused=False: tq_decode then tq_decode_reduce (partials in `partials` or
    allocated here); fused=True: tq_decode_fused with `workspace` (a zero-filled
    one is allocated here when None).

    q bf16 [S][Hq][128]; k_cache/v_cache uint8 (e4m3fn codes) [NB][Hkv][BS][128]
    (kv_layout "head") or [NB][BS][Hkv][128] ("slot", the page's data-region order);
    kv_scales fp32 [NB][Hkv][2][BS]; block_tables/seq_lens int32.
    ``max_seq_len`` (an upper bound of seq_lens) is read from seq_lens when not
    given, which synchronizes the stream; under graph capture it is the block
    table's capacity (max_blocks_per_seq * BS) instead, so that nothing is read
    back and the captured launches serve any lengths up to it.
    ``num_partitions`` defaults to ceil(max_seq_len / (256 * G)).
    ``stream``: a torch stream or raw hipStream_t (None: the current stream); the
    temporaries allocated here are allocated on it."""
    with _on_stream(stream):
        return _decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, num_partitions,
                       tile_groups_per_partition, softmax_scale, max_seq_len, partials, out, fused,
                       workspace, kv_layout, stream)


def _decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, num_partitions,
            tile_groups_per_partition, softmax_scale, max_seq_len, partials, out, fused, workspace,
            kv_layout, stream):
    S, Hq, D = q.shape
    _layout(kv_layout)
    if kv_layout == "head":
        NB, Hkv, BS, Dk = k_cache.shape
    else:
        NB, BS, Hkv, Dk = k_cache.shape
    if D != HEAD_DIM or Dk != HEAD_DIM or Hq % Hkv:
        raise ValueError("head_dim must be 128 and num_q_heads a multiple of num_kv_heads")
    QG = Hq // Hkv
    G = int(tile_groups_per_partition)
    if max_seq_len is None:
        if torch.cuda.is_current_stream_capturing():
            max_seq_len = int(block_tables.shape[1]) * BS
        else:
            max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    if num_partitions is None:
        num_partitions = max(1, -(-int(max_seq_len) // (TOKENS_PER_TILE_GROUP * G)))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((S, Hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    if fused:
        if workspace is None:
            workspace = alloc_fused_workspace(S, Hkv, QG, max_seq_len, q.device)
        tq_decode_fused(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, out, Hkv, QG, BS, G,
                        softmax_scale, num_partitions=num_partitions, max_seq_len=max_seq_len,
                        num_blocks=NB, workspace=workspace, kv_layout=kv_layout, stream=stream)
        return out
    if partials is None:
        partials = alloc_partials(S, Hkv, num_partitions, QG, q.device)
    tq_decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, partials, Hkv, QG, BS, G,
              softmax_scale, num_partitions=num_partitions, max_seq_len=max_seq_len,
              num_blocks=NB, kv_layout=kv_layout, stream=stream)
    tq_decode_reduce(partials, seq_lens, out, Hkv, QG, G, num_partitions=num_partitions,
                     max_seq_len=max_seq_len, stream=stream)
    return out
