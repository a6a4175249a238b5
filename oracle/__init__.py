"""fp64 CPU oracle for paged grouped-query decode attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the library's product
path never does.  It wraps ``oracle.c`` (plain C, fp64), which shares no code
with the HIP path.  What it computes follows the page
"vllm.v1.attention.ops.flydsl_kernels.tq_decode" (build_tq_decode_module and
the STEPs of tq_decode_kernel); the comment block of ``oracle.c`` states the
definition and the readings taken where that page is silent.

Array conventions (numpy, C-contiguous):
  q_bits        uint16 [S][Hkv*QG][D]   bfloat16 bit patterns
  k_codes       uint8  [NB][Hkv][BS][D] OCP e4m3fn codes (layout "head"), or
                       [NB][BS][Hkv][D] (layout "slot", the page's data-region order)
  v_codes       uint8  the same as k_codes
  kv_scales     float32 [NB][Hkv][2][BS] (field 0 = K, field 1 = V)
  block_tables  int32  [S][max_blocks_per_seq]
  seq_lens      int32  [S]

4-bit record format (decode_tq4):
  tq4_cache     uint8  [NB][Hkv*BS*D + Hkv*3*BS*2] data rows [Hkv][BS][D] (K indices in
                the first D/2 bytes, V indices in the last D/2; dim d = byte d/2, low
                nibble for even d), then fp16 meta [Hkv][3][BS] (K norm, V scale, V zero)
  centroids     float32 [16]
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_OK, ORC_ERR_ARGS, ORC_ERR_BLOCK, ORC_ERR_NOMEM = 0, 1, 2, 3
# Order of the K / V rows inside a cache block: head-major [Hkv][BS] or slot-major [BS][Hkv]
# (the page's data region).
LAYOUTS = {"head": 0, "slot": 1}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or a test's mutated copy)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.orc_dec_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.orc_dec_e4m3fn.restype = ctypes.c_double
        lib.orc_dec_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_dec_bf16.restype = ctypes.c_double
        lib.orc_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                   ctypes.c_float, i32, P, i32, P, i32]
        lib.orc_decode.restype = ctypes.c_int
        lib.orc_partials.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_float, i32, i32, i32, P, P, P]
        lib.orc_partials.restype = ctypes.c_int
        lib.orc_merge.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, P]
        lib.orc_merge.restype = ctypes.c_int
        lib.orc_enc_e4m3fn.argtypes = [ctypes.c_float]
        lib.orc_enc_e4m3fn.restype = ctypes.c_uint8
        lib.orc_kv_write.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P]
        lib.orc_kv_write.restype = ctypes.c_int
        lib.orc_dec_f16.argtypes = [ctypes.c_uint16]
        lib.orc_dec_f16.restype = ctypes.c_double
        lib.orc_decode_tq4.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, i32, P, i32, P, i32]
        lib.orc_decode_tq4.restype = ctypes.c_int
        lib.orc_dequant_tq4.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P]
        lib.orc_dequant_tq4.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def decode(self, q_bits, k_codes, v_codes, kv_scales, block_tables, seq_lens, softmax_scale,
               units=None, nthreads: int = 1, layout: str = "head") -> np.ndarray:
        """Unsplit decode attention in fp64.  ``layout``: "head" (codes [NB][Hkv][BS][D]) or
        "slot" ([NB][BS][Hkv][D], the page's data-region order).

        Returns [S][Hkv*QG][D] when ``units`` is None, else [len(units)][QG][D]
        for the listed (s, h) pairs."""
        q, k, v, sc, bt, sl, (S, Hkv, QG, D, BS, NB, MB) = _problem(
            q_bits, k_codes, v_codes, kv_scales, block_tables, seq_lens, layout)
        if units is None:
            u = None
            n = S * Hkv
        else:
            u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
            n = u.shape[0]
        out = np.empty((n, QG, D), dtype=np.float64)
        rc = self.lib.orc_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(sc), _ptr(bt), _ptr(sl), S, Hkv, QG,
                                 D, BS, NB, MB, float(softmax_scale), LAYOUTS[layout],
                                 None if u is None else _ptr(u), n, _ptr(out), int(nthreads))
        if rc:
            raise OracleError("orc_decode failed with code %d" % rc)
        if units is None:
            return out.reshape(S, Hkv * QG, D)
        return out

    def partials(self, q_bits, k_codes, v_codes, kv_scales, block_tables, seq_lens, softmax_scale,
                 num_partitions: int, partition_tokens: int, layout: str = "head"):
        """Split-K partials (o [S][Hkv][P][QG][D], m, l [S][Hkv][P][QG]); dead entries are NaN."""
        q, k, v, sc, bt, sl, (S, Hkv, QG, D, BS, NB, MB) = _problem(
            q_bits, k_codes, v_codes, kv_scales, block_tables, seq_lens, layout)
        P, E = int(num_partitions), int(partition_tokens)
        o = np.full((S, Hkv, P, QG, D), np.nan)
        m = np.full((S, Hkv, P, QG), np.nan)
        l = np.full((S, Hkv, P, QG), np.nan)
        rc = self.lib.orc_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(sc), _ptr(bt), _ptr(sl), S, Hkv,
                                   QG, D, BS, NB, MB, float(softmax_scale), LAYOUTS[layout], P, E,
                                   _ptr(o), _ptr(m), _ptr(l))
        if rc:
            raise OracleError("orc_partials failed with code %d" % rc)
        return o, m, l

    def merge(self, o, m, l, seq_lens, partition_tokens: int) -> np.ndarray:
        """Log-sum-exp merge of partials into [S][Hkv*QG][D]."""
        o = np.ascontiguousarray(o, dtype=np.float64)
        m = np.ascontiguousarray(m, dtype=np.float64)
        l = np.ascontiguousarray(l, dtype=np.float64)
        sl = _np(seq_lens, np.int32)
        S, Hkv, P, QG, D = o.shape
        out = np.empty((S, Hkv * QG, D), dtype=np.float64)
        rc = self.lib.orc_merge(_ptr(o), _ptr(m), _ptr(l), _ptr(sl), S, Hkv, QG, D, P,
                                int(partition_tokens), _ptr(out))
        if rc:
            raise OracleError("orc_merge failed with code %d" % rc)
        return out

    def decode_tq4(self, q_bits, tq4_cache, centroids, block_tables, seq_lens, softmax_scale,
                   num_kv_heads: int, kv_block_size: int, units=None, nthreads: int = 1,
                   layout: str = "head") -> np.ndarray:
        """Unsplit decode attention over the 4-bit record format, in fp64 (``layout``: the
        order of a block's data rows, "head" [Hkv][BS][D] or "slot" [BS][Hkv][D]).  Returns
        [S][Hkv*QG][D], or [len(units)][QG][D] for the listed (s, h) pairs."""
        q = _np(q_bits, np.uint16)
        cache = _np(tq4_cache, np.uint8)
        cent = _np(centroids, np.float32)
        bt = _np(block_tables, np.int32)
        sl = _np(seq_lens, np.int32)
        S, Hq, D = q.shape
        Hkv, BS = int(num_kv_heads), int(kv_block_size)
        QG = Hq // Hkv
        NB = cache.shape[0]
        if Hq % Hkv or cache.reshape(NB, -1).shape[1] != Hkv * BS * D + Hkv * 3 * BS * 2 \
                or cent.shape != (16,) or bt.shape[0] != S or sl.shape != (S,):
            raise OracleError("inconsistent shapes")
        if units is None:
            u = None
            n = S * Hkv
        else:
            u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
            n = u.shape[0]
        out = np.empty((n, QG, D), dtype=np.float64)
        rc = self.lib.orc_decode_tq4(_ptr(q), _ptr(cache), _ptr(cent), _ptr(bt), _ptr(sl), S, Hkv, QG,
                                     D, BS, NB, bt.shape[1], float(softmax_scale), LAYOUTS[layout],
                                     None if u is None else _ptr(u), n, _ptr(out), int(nthreads))
        if rc:
            raise OracleError("orc_decode_tq4 failed with code %d" % rc)
        return out.reshape(S, Hkv * QG, D) if units is None else out

    def dequant_tq4(self, tq4_cache, centroids, num_kv_heads: int, head_dim: int,
                    kv_block_size: int, block: int, head: int, slot: int, layout: str = "head"):
        """The dequantized K and V rows (fp64 [D] each) of one (block, head, slot)."""
        cache = _np(tq4_cache, np.uint8)
        cent = _np(centroids, np.float32)
        k = np.empty(head_dim, dtype=np.float64)
        v = np.empty(head_dim, dtype=np.float64)
        rc = self.lib.orc_dequant_tq4(_ptr(cache), _ptr(cent), int(num_kv_heads), int(head_dim),
                                      int(kv_block_size), LAYOUTS[layout], int(block), int(head),
                                      int(slot), _ptr(k), _ptr(v))
        if rc:
            raise OracleError("orc_dequant_tq4 failed with code %d" % rc)
        return k, v

    def dec_f16(self, bits) -> np.ndarray:
        """Decode IEEE fp16 bit patterns to float64 (closed form in oracle.c)."""
        b = _np(bits, np.uint16)
        flat = np.array([self.lib.orc_dec_f16(int(x)) for x in b.reshape(-1)], dtype=np.float64)
        return flat.reshape(b.shape)

    def dec_e4m3fn(self, codes) -> np.ndarray:
        """Decode OCP e4m3fn codes to float64 (closed form in oracle.c)."""
        table = np.array([self.lib.orc_dec_e4m3fn(c) for c in range(256)], dtype=np.float64)
        return table[_np(codes, np.uint8)]

    def dec_bf16(self, bits) -> np.ndarray:
        """Decode bfloat16 bit patterns to float64."""
        b = _np(bits, np.uint16)
        flat = np.array([self.lib.orc_dec_bf16(int(x)) for x in b.reshape(-1)], dtype=np.float64)
        return flat.reshape(b.shape)

    def enc_e4m3fn(self, values) -> np.ndarray:
        """Nearest e4m3fn codes (ties to even, saturating) of fp32 values."""
        v = np.asarray(values, dtype=np.float32)
        flat = np.array([self.lib.orc_enc_e4m3fn(float(x)) for x in v.reshape(-1)], dtype=np.uint8)
        return flat.reshape(v.shape)

    def kv_write(self, k_new_bits, v_new_bits, slot_mapping, k_cache, v_cache, kv_scales,
                 layout: str = "head"):
        """Quantize and scatter new K/V rows into copies of the cache arrays; returns them.
        k_new/v_new: bf16 bits [T][Hkv][D]; slot_mapping int32 [T] (-1: skip); the caches
        [NB][Hkv][BS][D] ("head") or [NB][BS][Hkv][D] ("slot")."""
        kn = _np(k_new_bits, np.uint16)
        vn = _np(v_new_bits, np.uint16)
        sm = _np(slot_mapping, np.int32)
        kc = _np(k_cache, np.uint8).copy()
        vc = _np(v_cache, np.uint8).copy()
        sc = _np(kv_scales, np.float32).copy()
        T, Hkv, D = kn.shape
        NB, Hkv2, BS, D2 = kc.shape if layout == "head" else _swap12(kc.shape)
        if vn.shape != kn.shape or Hkv2 != Hkv or D2 != D or sm.shape != (T,) or vc.shape != kc.shape \
                or sc.shape != (NB, Hkv, 2, BS):
            raise OracleError("inconsistent shapes")
        rc = self.lib.orc_kv_write(_ptr(kn), _ptr(vn), _ptr(sm), T, Hkv, D, BS, NB, LAYOUTS[layout],
                                   _ptr(kc), _ptr(vc), _ptr(sc))
        if rc:
            raise OracleError("orc_kv_write failed with code %d" % rc)
        return kc, vc, sc


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def build_variant(source_text: str, out_path: str) -> Oracle:
    """Compile a given C source text (e.g. a mutated copy of oracle.c) and load it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-w", "-o",
                    out_path, src, "-lm", "-lpthread"], check=True)
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _np(x, dtype):
    """torch tensor (CPU) or array -> C-contiguous numpy array of `dtype` (bit view for bf16)."""
    try:
        import torch  # noqa: WPS433
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            elif x.dtype == torch.float8_e4m3fn:
                x = x.view(torch.uint8)
            x = x.numpy()
    except ImportError:
        pass
    x = np.asarray(x)
    if x.dtype != np.dtype(dtype):
        if x.dtype.itemsize == np.dtype(dtype).itemsize and x.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
            x = x.view(dtype)
        else:
            x = x.astype(dtype)
    return np.ascontiguousarray(x)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _swap12(shape):
    return (shape[0], shape[2], shape[1], shape[3])


def _problem(q_bits, k_codes, v_codes, kv_scales, block_tables, seq_lens, layout="head"):
    q = _np(q_bits, np.uint16)
    k = _np(k_codes, np.uint8)
    v = _np(v_codes, np.uint8)
    sc = _np(kv_scales, np.float32)
    bt = _np(block_tables, np.int32)
    sl = _np(seq_lens, np.int32)
    if layout not in LAYOUTS:
        raise OracleError(f"layout must be one of {sorted(LAYOUTS)}")
    NB, Hkv, BS, D = k.shape if layout == "head" else _swap12(k.shape)
    S, Hq, Dq = q.shape
    if v.shape != k.shape or sc.shape != (NB, Hkv, 2, BS) or Dq != D or Hq % Hkv:
        raise OracleError("inconsistent shapes")
    if bt.ndim != 2 or bt.shape[0] != S or sl.shape != (S,):
        raise OracleError("inconsistent block table / seq_lens shapes")
    return q, k, v, sc, bt, sl, (S, Hkv, Hq // Hkv, D, BS, NB, bt.shape[1])


def decode(*a, **k):
    return default().decode(*a, **k)


def partials(*a, **k):
    return default().partials(*a, **k)


def merge(*a, **k):
    return default().merge(*a, **k)


def dec_e4m3fn(codes):
    return default().dec_e4m3fn(codes)


def dec_bf16(bits):
    return default().dec_bf16(bits)


def enc_e4m3fn(values):
    return default().enc_e4m3fn(values)


def kv_write(*a, **k):
    return default().kv_write(*a, **k)


def decode_tq4(*a, **k):
    return default().decode_tq4(*a, **k)


def dequant_tq4(*a, **k):
    return default().dequant_tq4(*a, **k)


def dec_f16(bits):
    return default().dec_f16(bits)
