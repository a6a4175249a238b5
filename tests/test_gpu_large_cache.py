"""Caches larger than 4 GiB: the blocks a decode reads, and the slots the writer
fills, sit above byte offsets 2^31 and 2^32 of the cache, so any 32-bit byte or
element offset in the kernels' address arithmetic would read or write the wrong
place.  The big caches are left unwritten except for the blocks the sequences
use; the oracle decodes a compact copy of those blocks through a renumbered block
table.  Needs an MI355X (about 13 GB of device memory)."""

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_amd as tq
import workloads
from gpu_util import ORACLE_THREADS, compare, say

pytestmark = pytest.mark.gpu

LENS = (1, 100, 777, 2049)


def spread_ids(n_used: int, nb_big: int, seed: int) -> np.ndarray:
    """n_used distinct block ids of a pool of nb_big: the top block, blocks just below and
    above the 2 GiB and 4 GiB marks of the pool, the rest drawn at random."""
    rng = np.random.default_rng(seed)
    fixed = [nb_big - 1, nb_big - 2, nb_big // 2 - 1, nb_big // 2, 0]
    rest = rng.choice(nb_big - 2, size=4 * n_used, replace=False)
    ids = list(dict.fromkeys(fixed + [int(x) for x in rest]))[:n_used]
    rng.shuffle(ids)
    return np.asarray(ids, dtype=np.int64)


def big_pool(block_bytes: int) -> int:
    """Blocks in a pool of just over 4 GiB + 64 MiB."""
    return -(-((1 << 32) + (64 << 20)) // block_bytes)


@pytest.mark.parametrize("bs", [16, 32])
def test_fp8_decode_above_4gib(bs):
    wl = workloads.small_workload(f"big{bs}", num_seqs=len(LENS), num_kv_heads=2, kv_block_size=bs,
                                  seq_lens=LENS, seed=700 + bs)
    c = workloads.make_inputs(wl, device="cpu", seq_lens=LENS)
    NB, Hkv = c.num_blocks, wl.num_kv_heads
    block_bytes = Hkv * bs * 128
    nb_big = big_pool(block_bytes)
    ids = spread_ids(NB, nb_big, seed=bs)
    assert ids.max() * block_bytes >= (1 << 32)
    say(f"[large cache] fp8 bs={bs} pool {nb_big} blocks ({nb_big * block_bytes / 2**30:.2f} GiB per cache)")
    ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.kv_scales, c.block_tables, c.seq_lens,
                        c.softmax_scale, nthreads=ORACLE_THREADS)
    idx = torch.from_numpy(ids).cuda()
    k = torch.empty((nb_big,) + tuple(c.k_cache.shape[1:]), dtype=torch.uint8, device="cuda")
    v = torch.empty_like(k)
    sc = torch.empty((nb_big,) + tuple(c.kv_scales.shape[1:]), dtype=torch.float32, device="cuda")
    k[idx] = c.k_cache.cuda()
    v[idx] = c.v_cache.cuda()
    sc[idx] = c.kv_scales.cuda()
    bt = torch.from_numpy(ids[c.block_tables.numpy()].astype(np.int32)).cuda()
    try:
        for fused in (False, True):
            out = tq.decode(c.q.cuda(), k, v, sc, bt, c.seq_lens.cuda(), max_seq_len=max(LENS),
                            softmax_scale=c.softmax_scale, fused=fused)
            torch.cuda.synchronize()
            compare(out, ref, f"fp8 above 4 GiB, bs={bs}, fused={fused}")
    finally:
        del k, v, sc
        torch.cuda.empty_cache()


def test_tq4_decode_above_4gib():
    bs = 16
    wl = workloads.small_workload("big_tq4", num_seqs=len(LENS), num_kv_heads=2, kv_block_size=bs,
                                  seq_lens=LENS, seed=751)
    c = workloads.make_inputs_tq4(wl, device="cpu", seq_lens=LENS)
    NB, Hkv = c.num_blocks, wl.num_kv_heads
    block_bytes = tq.tq4_block_bytes(Hkv, bs)
    nb_big = big_pool(block_bytes)
    ids = spread_ids(NB, nb_big, seed=5)
    assert ids.max() * block_bytes >= (1 << 32)
    say(f"[large cache] 4-bit bs={bs} pool {nb_big} blocks ({nb_big * block_bytes / 2**30:.2f} GiB)")
    ref = oracle.decode_tq4(c.q, c.cache, c.centroids, c.block_tables, c.seq_lens, c.softmax_scale,
                            Hkv, bs)
    cache = torch.empty((nb_big, block_bytes), dtype=torch.uint8, device="cuda")
    cache[torch.from_numpy(ids).cuda()] = c.cache.cuda()
    bt = torch.from_numpy(ids[c.block_tables.numpy()].astype(np.int32)).cuda()
    try:
        for fused in (False, True):
            out = tq.decode_tq4(c.q.cuda(), cache, c.centroids.cuda(), bt, c.seq_lens.cuda(),
                                num_kv_heads=Hkv, kv_block_size=bs, max_seq_len=max(LENS),
                                softmax_scale=c.softmax_scale, fused=fused)
            torch.cuda.synchronize()
            compare(out, ref, f"4-bit above 4 GiB, fused={fused}")
    finally:
        del cache
        torch.cuda.empty_cache()


def test_kv_write_above_4gib():
    """The writer's slots in the top blocks of a pool of over 4 GiB: codes and scales bit for
    bit against the oracle's writer on a compact copy of the touched blocks."""
    Hkv, bs, T = 2, 32, 96
    block_bytes = Hkv * bs * 128
    nb_big = big_pool(block_bytes)
    ids = np.asarray([nb_big - 1, nb_big - 3, nb_big // 2], dtype=np.int64)
    m = len(ids)
    rng = np.random.default_rng(17)
    kc = torch.from_numpy(rng.integers(0, 256, size=(m, Hkv, bs, 128), dtype=np.uint8))
    vc = torch.from_numpy(rng.integers(0, 256, size=(m, Hkv, bs, 128), dtype=np.uint8))
    sc = torch.from_numpy(rng.uniform(1, 2, size=(m, Hkv, 2, bs)).astype(np.float32))
    local = rng.permutation(m * bs)[:T].astype(np.int64)        # slots of the compact pool
    big_slots = (ids[local // bs] * bs + local % bs).astype(np.int32)
    g = torch.Generator().manual_seed(17)
    rows = torch.randn((2, T, Hkv, 128), generator=g).to(torch.bfloat16)
    ref_k, ref_v, ref_s = oracle.kv_write(rows[0], rows[1], local.astype(np.int32), kc, vc, sc)
    say(f"[large cache] kv_write into the top blocks of a {nb_big * block_bytes / 2**30:.2f} GiB pool")
    idx = torch.from_numpy(ids).cuda()
    k = torch.empty((nb_big, Hkv, bs, 128), dtype=torch.uint8, device="cuda")
    v = torch.empty_like(k)
    s = torch.empty((nb_big, Hkv, 2, bs), dtype=torch.float32, device="cuda")
    k[idx], v[idx], s[idx] = kc.cuda(), vc.cuda(), sc.cuda()
    try:
        tq.tq_kv_write(rows[0].cuda(), rows[1].cuda(), torch.from_numpy(big_slots).cuda(), k, v, s)
        torch.cuda.synchronize()
        assert np.array_equal(k[idx].cpu().numpy(), ref_k), "K codes differ from the oracle"
        assert np.array_equal(v[idx].cpu().numpy(), ref_v), "V codes differ from the oracle"
        assert np.array_equal(s[idx].cpu().numpy().view(np.uint32), ref_s.view(np.uint32)), \
            "scales differ from the oracle"
    finally:
        del k, v, s
        torch.cuda.empty_cache()
