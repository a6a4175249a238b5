"""Seeded synthetic inputs for paged grouped-query decode attention.

This module only draws inputs: queries, the fp8-quantized paged K/V cache with
its per-(token, kv head) scales, block tables and sequence lengths.  It holds
none of the attention arithmetic, so both the HIP path and the fp64 oracle can
consume what it produces without sharing code with each other.

Recipe (the same for every workload):
  * every random number comes from one counter-based generator written here
    (no library RNG): splitmix64 (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; the finalizer constants of
    Vigna's public reference code) applied to key + (i + 1) * 0x9E3779B97F4A7C15
    for the i-th number of a stream, with one key per (seed, stream);
    uniforms take the top 53 bits, N(0, 1) values the Box-Muller transform of
    two uniforms (numbers 2k and 2k + 1 give value k).  The 64-bit stream is
    the same bits on any device; the normals go through fp64 log / sqrt / cos,
    whose last-bit rounding may differ between devices;
  * streams: the sequence lengths (uniform integers), the permutation of the
    physical block pool (an argsort of random keys), the outlier channels (the
    first of another argsort), q, K and V (one normal per element, in the
    element order of [S][Hq][D] and [NB][Hkv][BS][D]);
  * q: bf16 round-to-nearest-even of N(0, 1), optionally with a seeded set of
    outlier (q head, dim) channels multiplied by 20 before rounding;
  * K, V: per (block, slot, kv head) row of head_dim values, scale =
    fp32(absmax / 448) and codes = e4m3fn(x / scale) rounded to nearest even
    (torch's cast, after clamping to +-448); an all-zero row has scale 0 and
    codes 0;
  * block tables: a random permutation of the pool handed out to the sequences
    in order, ceil(L / BS) blocks each; unused table entries are 0.

Layouts (all C-contiguous):
  q             bf16   [S][Hkv*QG][D]
  k_cache       uint8  [NB][Hkv][BS][D]  (e4m3fn codes, kv_layout "head": one (block, kv head)
                                          slice contiguous), or [NB][BS][Hkv][D] ("slot": the
                                          page's data-region order; the same values, permuted)
  v_cache       uint8  the same as k_cache
  kv_scales     fp32   [NB][Hkv][2][BS]  (field 0 = K, field 1 = V)
  block_tables  int32  [S][max_blocks_per_seq]
  seq_lens      int32  [S]
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_E4M3FN_MAX = 448.0
TOKENS_PER_TILE_GROUP = 256  # 16 tiles of 16 tokens
SLAB_BLOCKS = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_kv_heads: int
    query_group_size: int
    kv_block_size: int
    seq_len_lo: int
    seq_len_hi: int
    tile_groups_per_partition: int
    max_blocks_per_seq: int
    seed: int
    head_dim: int = 128
    num_partitions: Optional[int] = None  # None: sized to the longest sequence
    num_blocks: Optional[int] = None  # None: exactly the blocks the sequences use
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    permute_pool: bool = True

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.query_group_size

    @property
    def partition_tokens(self) -> int:
        return TOKENS_PER_TILE_GROUP * self.tile_groups_per_partition


def _W(**kw) -> Workload:
    return Workload(**kw)


# The five workloads: shapes, length mixes and data distributions of the decode
# configurations this library is specified against.
WORKLOADS = {
    "w1_tiny": _W(name="w1_tiny", num_seqs=1, num_kv_heads=1, query_group_size=8, kv_block_size=16,
                  seq_len_lo=256, seq_len_hi=256, tile_groups_per_partition=1,
                  max_blocks_per_seq=16, num_blocks=16, num_partitions=1, seed=0x5EED0001),
    "w2_s32_ctx4k": _W(name="w2_s32_ctx4k", num_seqs=32, num_kv_heads=8, query_group_size=8,
                       kv_block_size=16, seq_len_lo=4096, seq_len_hi=4096,
                       tile_groups_per_partition=1, max_blocks_per_seq=256, num_blocks=8192,
                       num_partitions=16, seed=0x5EED0002),
    "w3_s64_ragged": _W(name="w3_s64_ragged", num_seqs=64, num_kv_heads=8, query_group_size=6,
                        kv_block_size=32, seq_len_lo=1024, seq_len_hi=8192,
                        tile_groups_per_partition=1, max_blocks_per_seq=256, seed=0x5EED0003),
    "w4_s128_ctx8k": _W(name="w4_s128_ctx8k", num_seqs=128, num_kv_heads=8, query_group_size=8,
                        kv_block_size=32, seq_len_lo=8192, seq_len_hi=8192,
                        tile_groups_per_partition=1, max_blocks_per_seq=256, num_blocks=32768,
                        num_partitions=32, seed=0x5EED0004),
    "w5_s16_long": _W(name="w5_s16_long", num_seqs=16, num_kv_heads=4, query_group_size=16,
                      kv_block_size=32, seq_len_lo=16384, seq_len_hi=40960,
                      tile_groups_per_partition=5, max_blocks_per_seq=1280, seed=0x5EED0005,
                      outlier_frac=0.01),
}


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    kv_scales: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    num_partitions: int
    num_blocks: int
    softmax_scale: float
    kv_layout: str = "head"

    def to(self, device) -> "Inputs":
        f = lambda t: t.to(device)  # noqa: E731
        return dataclasses.replace(self, q=f(self.q), k_cache=f(self.k_cache), v_cache=f(self.v_cache),
                                   kv_scales=f(self.kv_scales), block_tables=f(self.block_tables),
                                   seq_lens=f(self.seq_lens))

    def with_layout(self, kv_layout: str) -> "Inputs":
        """The same inputs with the cache rows in the other order (a permuted copy)."""
        if kv_layout == self.kv_layout:
            return self
        swap = lambda t: t.permute(0, 2, 1, 3).contiguous()  # noqa: E731
        return dataclasses.replace(self, k_cache=swap(self.k_cache), v_cache=swap(self.v_cache),
                                   kv_layout=kv_layout)

    def kv_bytes(self) -> int:
        """Bytes of live K/V codes plus scales: sum over sequences and kv heads of L * (2*D + 8)."""
        D = self.wl.head_dim
        return int(self.seq_lens.to(torch.int64).sum().item()) * self.wl.num_kv_heads * (2 * D + 8)


# ----------------------------------------------------------------------------
# The counter-based generator (splitmix64 on a counter; see the recipe above).
# ----------------------------------------------------------------------------

SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
SPLITMIX_M1 = 0xBF58476D1CE4E5B9
SPLITMIX_M2 = 0x94D049BB133111EB
_U64 = (1 << 64) - 1
STREAMS = {"lens": 1, "pool": 2, "outliers": 3, "q": 4, "k": 5, "v": 6, "writer": 7, "poison": 8}


def _i64(c: int) -> int:
    """A 64-bit pattern as the int64 value with the same bits."""
    c &= _U64
    return c - (1 << 64) if c >> 63 else c


def _shr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """The splitmix64 finalizer on int64 bit patterns (multiplications wrap mod 2^64)."""
    z = (z ^ _shr(z, 30)) * _i64(SPLITMIX_M1)
    z = (z ^ _shr(z, 27)) * _i64(SPLITMIX_M2)
    return z ^ _shr(z, 31)


def mix64_int(z: int) -> int:
    """The same finalizer on a Python integer."""
    z &= _U64
    z = ((z ^ (z >> 30)) * SPLITMIX_M1) & _U64
    z = ((z ^ (z >> 27)) * SPLITMIX_M2) & _U64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: str) -> int:
    """The key of one stream of a seed."""
    return mix64_int((seed << 8) + STREAMS[stream])


def random_bits(key: int, start: int, n: int, device) -> torch.Tensor:
    """Numbers start .. start + n - 1 of the stream with this key, as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return mix64(i * _i64(SPLITMIX_GAMMA) + _i64(key))


def random_uniform(key: int, start: int, n: int, device) -> torch.Tensor:
    """Uniforms in (0, 1), fp64: (top 53 bits + 0.5) / 2^53."""
    return (_shr(random_bits(key, start, n, device), 11).to(torch.float64) + 0.5) * 2.0 ** -53


def random_normal(key: int, start: int, n: int, device) -> torch.Tensor:
    """N(0, 1) values start .. start + n - 1, fp64: value k is sqrt(-2 ln u1) cos(2 pi u2)
    with u1, u2 the uniforms 2k and 2k + 1."""
    u = random_uniform(key, 2 * start, 2 * n, device).view(n, 2)
    return torch.sqrt(-2.0 * torch.log(u[:, 0])) * torch.cos(2.0 * math.pi * u[:, 1])


def random_permutation(key: int, n: int, device="cpu") -> torch.Tensor:
    """A permutation of 0 .. n-1 (int64): the stable argsort of n random keys."""
    b = random_bits(key, 0, n, device)
    return torch.sort(_shr(b, 1), stable=True).indices


def random_ints(key: int, start: int, n: int, hi: int) -> np.ndarray:
    """n integers in [0, hi) (int64, CPU): the top 53 bits of each number scaled to hi."""
    u = random_uniform(key, start, n, "cpu").numpy()
    return np.minimum(np.floor(u * hi), hi - 1).astype(np.int64)


def draw_seq_lens(wl: Workload) -> np.ndarray:
    if wl.seq_len_lo == wl.seq_len_hi:
        return np.full(wl.num_seqs, wl.seq_len_lo, dtype=np.int32)
    span = wl.seq_len_hi - wl.seq_len_lo + 1
    return (wl.seq_len_lo + random_ints(stream_key(wl.seed, "lens"), 0, wl.num_seqs, span)).astype(np.int32)


def quantize_rows(x: torch.Tensor):
    """fp32 [..., D] -> (e4m3fn codes uint8 [..., D], fp32 scale [...]) with scale = absmax / 448."""
    absmax = x.abs().amax(dim=-1)
    scale = absmax / FP8_E4M3FN_MAX
    div = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = (x / div.unsqueeze(-1)).clamp_(-FP8_E4M3FN_MAX, FP8_E4M3FN_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_inputs(wl: Workload, device="cpu", seq_lens=None, num_partitions=None,
                softmax_scale: Optional[float] = None, _skip_cache: bool = False,
                kv_layout: str = "head") -> Inputs:
    """Draw the inputs of workload `wl` on `device` (deterministic per device); kv_layout
    "slot" gives the same values with the cache rows slot-major.
    _skip_cache: leave the fp8 cache empty (for the 4-bit format's generator)."""
    dev = torch.device(device)
    sl = draw_seq_lens(wl) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    S, Hkv, QG, D, BS = wl.num_seqs, wl.num_kv_heads, wl.query_group_size, wl.head_dim, wl.kv_block_size
    assert sl.shape == (S,)
    need = [-(-int(L) // BS) for L in sl]
    NB = wl.num_blocks if wl.num_blocks is not None else max(1, sum(need))
    assert NB >= sum(need), "block pool smaller than the sequences need"
    assert max(need) <= wl.max_blocks_per_seq
    pool = (random_permutation(stream_key(wl.seed, "pool"), NB).numpy().astype(np.int32)
            if wl.permute_pool else np.arange(NB, dtype=np.int32))
    bt = np.zeros((S, wl.max_blocks_per_seq), dtype=np.int32)
    pos = 0
    for s in range(S):
        bt[s, :need[s]] = pool[pos:pos + need[s]]
        pos += need[s]
    if num_partitions is None:
        num_partitions = wl.num_partitions
    if num_partitions is None:
        num_partitions = max(1, -(-int(sl.max()) // wl.partition_tokens))

    q = random_normal(stream_key(wl.seed, "q"), 0, S * Hkv * QG * D, dev).float()
    q = q.view(S, Hkv * QG, D)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * Hkv * QG * D))
        chans = random_permutation(stream_key(wl.seed, "outliers"), Hkv * QG * D)[:n_out]
        mult = torch.ones(Hkv * QG * D, dtype=torch.float32)
        mult[chans] = wl.outlier_mult
        q = q * mult.view(1, Hkv * QG, D).to(dev)
    q = q.to(torch.bfloat16)

    if _skip_cache:
        if softmax_scale is None:
            softmax_scale = float(np.float32(1.0 / math.sqrt(D)))
        empty = torch.empty(0, dtype=torch.uint8, device=dev)
        return Inputs(wl=wl, q=q, k_cache=empty, v_cache=empty, kv_scales=empty,
                      block_tables=torch.from_numpy(bt).to(dev), seq_lens=torch.from_numpy(sl).to(dev),
                      num_partitions=int(num_partitions), num_blocks=NB, softmax_scale=softmax_scale)
    k_codes = torch.empty((NB, Hkv, BS, D), dtype=torch.uint8, device=dev)
    v_codes = torch.empty((NB, Hkv, BS, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((NB, Hkv, 2, BS), dtype=torch.float32, device=dev)
    row = Hkv * BS * D  # elements per cache block
    for b0 in range(0, NB, SLAB_BLOCKS):
        b1 = min(NB, b0 + SLAB_BLOCKS)
        for field, (stream, dst) in enumerate((("k", k_codes), ("v", v_codes))):
            x = random_normal(stream_key(wl.seed, stream), b0 * row, (b1 - b0) * row, dev).float()
            x = x.view(b1 - b0, Hkv, BS, D)
            codes, sc = quantize_rows(x)
            dst[b0:b1] = codes
            scales[b0:b1, :, field, :] = sc
            del x, codes, sc
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(D)))
    inp = Inputs(wl=wl, q=q, k_cache=k_codes, v_cache=v_codes, kv_scales=scales,
                 block_tables=torch.from_numpy(bt).to(dev), seq_lens=torch.from_numpy(sl).to(dev),
                 num_partitions=int(num_partitions), num_blocks=NB, softmax_scale=softmax_scale)
    if kv_layout != "head":
        del k_codes, v_codes
        inp = inp.with_layout(kv_layout)
    return inp


def small_workload(name="small", num_seqs=3, num_kv_heads=2, query_group_size=8, kv_block_size=16,
                   seq_lens=(1, 17, 300), tile_groups_per_partition=1, max_blocks_per_seq=None,
                   extra_blocks=3, seed=1234, outlier_frac=0.0) -> Workload:
    """A small workload for parity sweeps: explicit lengths via make_inputs(seq_lens=...)."""
    BS = kv_block_size
    mb = max_blocks_per_seq or max(1, max(-(-int(L) // BS) for L in seq_lens) + 2)
    nb = sum(-(-int(L) // BS) for L in seq_lens) + extra_blocks
    return Workload(name=name, num_seqs=num_seqs, num_kv_heads=num_kv_heads,
                    query_group_size=query_group_size, kv_block_size=BS, seq_len_lo=0,
                    seq_len_hi=0, tile_groups_per_partition=tile_groups_per_partition,
                    max_blocks_per_seq=mb, seed=seed, num_blocks=max(1, nb),
                    outlier_frac=outlier_frac)


def poison(inp: Inputs, seed: int = 99) -> Inputs:
    """Copy of `inp` with garbage wherever a correct reader must not look.

    * cache slots past each sequence's length inside its last block: K/V codes
      0x7F (NaN) and NaN scales;
    * block-table entries past ceil(L / BS): other valid block ids of the pool
      (never out of range, so a wrong reader gives wrong numbers, not a fault).
    """
    key, used = stream_key(seed, "poison"), 0
    k = inp.k_cache.clone()
    v = inp.v_cache.clone()
    sc = inp.kv_scales.clone()
    bt = inp.block_tables.cpu().numpy().copy()
    sl = inp.seq_lens.cpu().numpy()
    BS = inp.wl.kv_block_size
    # the slots of a block: dim 2 of a head-major cache, dim 1 of a slot-major one
    kh = k if inp.kv_layout == "head" else k.transpose(1, 2)
    vh = v if inp.kv_layout == "head" else v.transpose(1, 2)
    for s, L in enumerate(sl):
        L = int(L)
        nb_used = -(-L // BS)
        if L % BS:
            b = int(bt[s, nb_used - 1])
            kh[b, :, L % BS:] = 0x7F
            vh[b, :, L % BS:] = 0x7F
            sc[b, :, :, L % BS:] = float("nan")
        tail = bt.shape[1] - nb_used
        if tail > 0:
            bt[s, nb_used:] = random_ints(key, used, tail, inp.num_blocks)
            used += tail
    return dataclasses.replace(inp, k_cache=k, v_cache=v, kv_scales=sc,
                               block_tables=torch.from_numpy(bt).to(inp.block_tables.device))


# ----------------------------------------------------------------------------
# The 4-bit record format (the "TQ" cache of page "vllm.v1.attention.ops.
# flydsl_kernels.tq_decode").  Layout of one cache block (uint8):
#   data rows [Hkv][BS][D]: per (kv head, slot) D bytes, the K indices in the
#     first D/2 (dim d in byte d/2, low nibble for even d), the V indices in
#     the last D/2;
#   meta [Hkv][3][BS] fp16: K norm, V scale, V zero point.
# Recipe: q as above (the query arrives already rotated: a rotation of an
# isotropic Gaussian is one); K rows x ~ N(0, 1) (the fp8 format's K stream): knorm = fp16(|x| / sqrt(D)),
# indices = nearest of the 16 centroids to x / knorm; V rows y ~ N(0, 1): zero
# = fp16(min y), scale = fp16((max y - min y) / 15), indices = round((y - zero)
# / scale) clamped to [0, 15].  The centroids are those of the 16-level
# Lloyd-Max quantizer of N(0, 1) (a plain fixed-point iteration, no RNG).
# ----------------------------------------------------------------------------

TQ4_META_FIELDS = 3


def tq4_block_bytes(num_kv_heads: int, kv_block_size: int, head_dim: int = 128) -> int:
    return num_kv_heads * kv_block_size * head_dim + num_kv_heads * TQ4_META_FIELDS * kv_block_size * 2


def lloyd_max_normal_16(iters: int = 200) -> np.ndarray:
    """Centroids (float32, ascending) of the 16-level Lloyd-Max quantizer of N(0, 1)."""
    phi = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)  # noqa: E731
    Phi = lambda x: 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))  # noqa: E731
    c = [-2.5 + 5.0 * j / 15 for j in range(16)]
    for _ in range(iters):
        b = [-math.inf] + [(c[j] + c[j + 1]) / 2 for j in range(15)] + [math.inf]
        c = []
        for j in range(16):
            lo, hi = b[j], b[j + 1]
            pl = 0.0 if lo == -math.inf else phi(lo)
            ph = 0.0 if hi == math.inf else phi(hi)
            mass = (1.0 if hi == math.inf else Phi(hi)) - (0.0 if lo == -math.inf else Phi(lo))
            c.append((pl - ph) / mass)
    return np.asarray(c, dtype=np.float32)


def pack_tq4(k_idx: torch.Tensor, v_idx: torch.Tensor, meta_bits: torch.Tensor,
             kv_layout: str = "head") -> torch.Tensor:
    """Indices uint8 [NB][Hkv][BS][D] (values 0..15) and fp16 meta bits int16
    [NB][Hkv][3][BS] -> cache uint8 [NB][block_bytes], the data rows in the order kv_layout
    names ("head" [Hkv][BS], "slot" [BS][Hkv])."""
    NB, Hkv, BS, D = k_idx.shape
    data = torch.empty((NB, Hkv, BS, D), dtype=torch.uint8, device=k_idx.device)
    data[..., :D // 2] = k_idx[..., 0::2] | (k_idx[..., 1::2] << 4)
    data[..., D // 2:] = v_idx[..., 0::2] | (v_idx[..., 1::2] << 4)
    if kv_layout != "head":
        data = data.permute(0, 2, 1, 3).contiguous()
    meta = meta_bits.contiguous().view(torch.uint8).reshape(NB, -1)
    return torch.cat([data.reshape(NB, -1), meta], dim=1).contiguous()


def quantize_tq4_rows(x: torch.Tensor, y: torch.Tensor, centroids: torch.Tensor):
    """K rows x and V rows y, fp32 [..., D] -> (K indices, V indices, fp16 meta [..., 3])."""
    D = x.shape[-1]
    knorm = (x.norm(dim=-1) / math.sqrt(D)).to(torch.float16)
    kn = knorm.float()
    u = x / torch.where(kn > 0, kn, torch.ones_like(kn)).unsqueeze(-1)
    mids = (centroids[:-1] + centroids[1:]) / 2
    k_idx = torch.bucketize(u.contiguous(), mids.contiguous()).to(torch.uint8)
    lo = y.amin(dim=-1)
    hi = y.amax(dim=-1)
    zero = lo.to(torch.float16)
    scale = ((hi - lo) / 15).to(torch.float16)
    sc = scale.float()
    div = torch.where(sc > 0, sc, torch.ones_like(sc)).unsqueeze(-1)
    v_idx = torch.round((y - zero.float().unsqueeze(-1)) / div).clamp_(0, 15).to(torch.uint8)
    v_idx = torch.where(sc.unsqueeze(-1) > 0, v_idx, torch.zeros_like(v_idx))
    meta = torch.stack([knorm, scale, zero], dim=-1)
    return k_idx, v_idx, meta


@dataclasses.dataclass
class InputsTq4:
    wl: Workload
    q: torch.Tensor            # bf16 [S][Hkv*QG][D], the rotated query
    cache: torch.Tensor        # uint8 [NB][block_bytes]
    centroids: torch.Tensor    # fp32 [16]
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    num_partitions: int
    num_blocks: int
    softmax_scale: float
    kv_layout: str = "head"

    def with_layout(self, kv_layout: str) -> "InputsTq4":
        """The same records with the data rows of every block in the other order."""
        if kv_layout == self.kv_layout:
            return self
        wl = self.wl
        Hkv, BS, D = wl.num_kv_heads, wl.kv_block_size, wl.head_dim
        NB = self.cache.shape[0]
        nd = Hkv * BS * D
        data = self.cache[:, :nd].reshape(NB, *((Hkv, BS) if self.kv_layout == "head" else (BS, Hkv)), D)
        data = data.permute(0, 2, 1, 3).reshape(NB, nd)
        return dataclasses.replace(self, cache=torch.cat([data, self.cache[:, nd:]], dim=1).contiguous(),
                                   kv_layout=kv_layout)

    def to(self, device) -> "InputsTq4":
        f = lambda t: t.to(device)  # noqa: E731
        return dataclasses.replace(self, q=f(self.q), cache=f(self.cache), centroids=f(self.centroids),
                                   block_tables=f(self.block_tables), seq_lens=f(self.seq_lens))

    def kv_bytes(self) -> int:
        """Bytes of live records: sum over sequences and kv heads of L * (D + 6)."""
        D = self.wl.head_dim
        return int(self.seq_lens.to(torch.int64).sum().item()) * self.wl.num_kv_heads * (D + 2 * TQ4_META_FIELDS)


def make_inputs_tq4(wl: Workload, device="cpu", seq_lens=None, num_partitions=None,
                    softmax_scale: Optional[float] = None, kv_layout: str = "head") -> InputsTq4:
    """Draw the 4-bit-format inputs of workload `wl` on `device` (same lengths, tables and q
    as make_inputs; the cache from the same K/V draws, quantized to the 4-bit record)."""
    dev = torch.device(device)
    base = make_inputs(wl, device=dev, seq_lens=seq_lens, num_partitions=num_partitions,
                       softmax_scale=softmax_scale, _skip_cache=True)
    S, Hkv, D, BS = wl.num_seqs, wl.num_kv_heads, wl.head_dim, wl.kv_block_size
    NB = base.num_blocks
    cent = torch.from_numpy(lloyd_max_normal_16()).to(dev)
    cache = torch.empty((NB, tq4_block_bytes(Hkv, BS, D)), dtype=torch.uint8, device=dev)
    row = Hkv * BS * D
    for b0 in range(0, NB, SLAB_BLOCKS):
        b1 = min(NB, b0 + SLAB_BLOCKS)
        x = random_normal(stream_key(wl.seed, "k"), b0 * row, (b1 - b0) * row, dev).float()
        y = random_normal(stream_key(wl.seed, "v"), b0 * row, (b1 - b0) * row, dev).float()
        x, y = x.view(b1 - b0, Hkv, BS, D), y.view(b1 - b0, Hkv, BS, D)
        k_idx, v_idx, meta = quantize_tq4_rows(x, y, cent)
        meta_bits = meta.view(torch.int16).permute(0, 1, 3, 2).contiguous()  # [b][Hkv][3][BS]
        cache[b0:b1] = pack_tq4(k_idx, v_idx, meta_bits, kv_layout)
        del x, y, k_idx, v_idx, meta, meta_bits
    return InputsTq4(wl=wl, q=base.q, cache=cache, centroids=cent, block_tables=base.block_tables,
                     seq_lens=base.seq_lens, num_partitions=base.num_partitions, num_blocks=NB,
                     softmax_scale=base.softmax_scale, kv_layout=kv_layout)


def poison_tq4(inp: InputsTq4, seed: int = 99) -> InputsTq4:
    """Copy of `inp` with garbage wherever a correct reader must not look: the records of
    slots past each sequence's length in its last block get random index bytes and NaN
    meta (fp16 0x7E00); block-table entries past ceil(L / BS) get other valid block ids."""
    key, used = stream_key(seed, "poison"), 0
    cache = inp.cache.clone()
    bt = inp.block_tables.cpu().numpy().copy()
    sl = inp.seq_lens.cpu().numpy()
    wl = inp.wl
    Hkv, BS, D = wl.num_kv_heads, wl.kv_block_size, wl.head_dim
    data_bytes = Hkv * BS * D
    for s, L in enumerate(sl):
        L = int(L)
        nb_used = -(-L // BS)
        if L % BS:
            b = int(bt[s, nb_used - 1])
            blk = cache[b]
            rows = blk[:data_bytes].view(Hkv, BS, D) if inp.kv_layout == "head" else \
                blk[:data_bytes].view(BS, Hkv, D).transpose(0, 1)
            n = Hkv * (BS - L % BS) * D
            rows[:, L % BS:] = torch.from_numpy(random_ints(key, used, n, 256).astype(np.uint8).reshape(
                Hkv, BS - L % BS, D)).to(cache.device)
            used += n
            meta = blk[data_bytes:].view(torch.int16).view(Hkv, TQ4_META_FIELDS, BS)
            meta[:, :, L % BS:] = 0x7E00
        tail = bt.shape[1] - nb_used
        if tail > 0:
            bt[s, nb_used:] = random_ints(key, used, tail, inp.num_blocks)
            used += tail
    return dataclasses.replace(inp, cache=cache,
                               block_tables=torch.from_numpy(bt).to(inp.block_tables.device))
