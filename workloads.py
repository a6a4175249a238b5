"""Seeded synthetic inputs for paged grouped-query decode attention.

This module only draws inputs: queries, the fp8-quantized paged K/V cache with
its per-(token, kv head) scales, block tables and sequence lengths.  It holds
none of the attention arithmetic, so both the HIP path and the fp64 oracle can
consume what it produces without sharing code with each other.

Recipe (the same for every workload):
  * numpy ``default_rng(seed)`` draws the sequence lengths, the permutation of
    the physical block pool and the outlier channels;
  * torch's generator (seed+1 for q, seed+2 for K, seed+3 for V), on the
    requested device, draws N(0, 1) values; K and V are drawn in slabs of at
    most ``SLAB_BLOCKS`` cache blocks, K slab then V slab;
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


def draw_seq_lens(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    if wl.seq_len_lo == wl.seq_len_hi:
        return np.full(wl.num_seqs, wl.seq_len_lo, dtype=np.int32)
    return rng.integers(wl.seq_len_lo, wl.seq_len_hi + 1, size=wl.num_seqs).astype(np.int32)


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
    rng = np.random.default_rng(wl.seed)
    sl = draw_seq_lens(wl, rng) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    S, Hkv, QG, D, BS = wl.num_seqs, wl.num_kv_heads, wl.query_group_size, wl.head_dim, wl.kv_block_size
    assert sl.shape == (S,)
    need = [-(-int(L) // BS) for L in sl]
    NB = wl.num_blocks if wl.num_blocks is not None else max(1, sum(need))
    assert NB >= sum(need), "block pool smaller than the sequences need"
    assert max(need) <= wl.max_blocks_per_seq
    pool = rng.permutation(NB).astype(np.int32) if wl.permute_pool else np.arange(NB, dtype=np.int32)
    bt = np.zeros((S, wl.max_blocks_per_seq), dtype=np.int32)
    pos = 0
    for s in range(S):
        bt[s, :need[s]] = pool[pos:pos + need[s]]
        pos += need[s]
    if num_partitions is None:
        num_partitions = wl.num_partitions
    if num_partitions is None:
        num_partitions = max(1, -(-int(sl.max()) // wl.partition_tokens))

    gq = torch.Generator(device=dev).manual_seed(wl.seed + 1)
    q = torch.randn((S, Hkv * QG, D), generator=gq, device=dev, dtype=torch.float32)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * Hkv * QG * D))
        chans = rng.choice(Hkv * QG * D, size=n_out, replace=False)
        mult = torch.ones(Hkv * QG * D, dtype=torch.float32)
        mult[torch.from_numpy(chans.astype(np.int64))] = wl.outlier_mult
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
    gk = torch.Generator(device=dev).manual_seed(wl.seed + 2)
    gv = torch.Generator(device=dev).manual_seed(wl.seed + 3)
    for b0 in range(0, NB, SLAB_BLOCKS):
        b1 = min(NB, b0 + SLAB_BLOCKS)
        for field, (gen, dst) in enumerate(((gk, k_codes), (gv, v_codes))):
            x = torch.randn((b1 - b0, Hkv, BS, D), generator=gen, device=dev, dtype=torch.float32)
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
    rng = np.random.default_rng(seed)
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
            bt[s, nb_used:] = rng.integers(0, inp.num_blocks, size=tail)
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
# isotropic Gaussian is one); K rows x ~ N(0, 1): knorm = fp16(|x| / sqrt(D)),
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
    gk = torch.Generator(device=dev).manual_seed(wl.seed + 2)
    gv = torch.Generator(device=dev).manual_seed(wl.seed + 3)
    for b0 in range(0, NB, SLAB_BLOCKS):
        b1 = min(NB, b0 + SLAB_BLOCKS)
        x = torch.randn((b1 - b0, Hkv, BS, D), generator=gk, device=dev, dtype=torch.float32)
        y = torch.randn((b1 - b0, Hkv, BS, D), generator=gv, device=dev, dtype=torch.float32)
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
    rng = np.random.default_rng(seed)
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
            rows[:, L % BS:] = torch.from_numpy(
                rng.integers(0, 256, size=(Hkv, BS - L % BS, D), dtype=np.uint8)).to(cache.device)
            meta = blk[data_bytes:].view(torch.int16).view(Hkv, TQ4_META_FIELDS, BS)
            meta[:, :, L % BS:] = 0x7E00
        tail = bt.shape[1] - nb_used
        if tail > 0:
            bt[s, nb_used:] = rng.integers(0, inp.num_blocks, size=tail)
    return dataclasses.replace(inp, cache=cache,
                               block_tables=torch.from_numpy(bt).to(inp.block_tables.device))
