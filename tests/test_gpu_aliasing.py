"""Block aliasing (prefix sharing): several sequences' block tables name the same physical
cache blocks.  The decode only reads the cache, so a table may point any number of sequences
at one block.  Checked on both cache formats and both paths against the fp64 oracle, and bit
for bit against a copy of the same data in which every shared block is duplicated so that no
two table entries name the same block.  Needs an MI355X."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_amd as tq
import workloads
from gpu_util import ORACLE_THREADS, PATHS, compare, gpu_decode, oracle_decode, say

pytestmark = pytest.mark.gpu

LENS = (700, 700, 300, 1000, 1, 520)


def alias_tables(bt: np.ndarray, BS: int) -> np.ndarray:
    """Tables with shared prefixes: sequence 1 shares its first 20 blocks with sequence 0,
    sequence 2 lies wholly inside sequence 0's first blocks (its last block partly used),
    sequence 3 shares 10 blocks with sequence 1 (so also with 0), sequence 4 reads sequence
    3's first block, sequence 5 reads the same block for all its entries (one block read many
    times over)."""
    bt = bt.copy()
    bt[1, :20] = bt[0, :20]
    n2 = -(-LENS[2] // BS)
    bt[2, :n2] = bt[0, :n2]
    bt[3, :10] = bt[1, :10]
    bt[4, 0] = bt[3, 0]
    n5 = -(-LENS[5] // BS)
    bt[5, :n5] = bt[5, 0]
    return bt


def dealias(bt: np.ndarray, BS: int, num_blocks: int):
    """(new table, source block of each new block id >= num_blocks): every table entry below a
    sequence's length that repeats a block already named gets a fresh block id."""
    bt = bt.copy()
    seen, extra = set(), []
    for s, L in enumerate(LENS):
        for j in range(-(-L // BS)):
            b = int(bt[s, j])
            if b in seen:
                bt[s, j] = num_blocks + len(extra)
                extra.append(b)
            else:
                seen.add(b)
    return bt, extra


def _fp8_inputs(bs, seed):
    wl = workloads.small_workload(name="alias", num_seqs=len(LENS), num_kv_heads=2,
                                  query_group_size=8, kv_block_size=bs, seq_lens=LENS, seed=seed)
    return workloads.make_inputs(wl, device="cuda", seq_lens=LENS, num_partitions=4)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [16, 32])
def test_fp8_aliased_blocks(bs, path):
    inp = _fp8_inputs(bs, 71 + bs)
    bt = alias_tables(inp.block_tables.cpu().numpy(), bs)
    aliased = dataclasses.replace(inp, block_tables=torch.from_numpy(bt).cuda())
    say(f"[aliasing] fp8 bs={bs} {path}")
    out = gpu_decode(aliased, path=path)
    compare(out, oracle_decode(aliased), f"fp8 aliased bs{bs} {path}")
    bt2, extra = dealias(bt, bs, inp.num_blocks)
    assert extra, "the tables must share blocks"
    src = torch.tensor(extra, dtype=torch.int64, device="cuda")
    flat = dataclasses.replace(
        inp, block_tables=torch.from_numpy(bt2).cuda(),
        k_cache=torch.cat([inp.k_cache, inp.k_cache[src]]).contiguous(),
        v_cache=torch.cat([inp.v_cache, inp.v_cache[src]]).contiguous(),
        kv_scales=torch.cat([inp.kv_scales, inp.kv_scales[src]]).contiguous(),
        num_blocks=inp.num_blocks + len(extra))
    ref = gpu_decode(flat, path=path)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [16, 32])
def test_tq4_aliased_blocks(bs, path):
    wl = workloads.small_workload(name="alias4", num_seqs=len(LENS), num_kv_heads=2,
                                  query_group_size=16, kv_block_size=bs, seq_lens=LENS,
                                  seed=81 + bs)
    inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=LENS, num_partitions=4)
    bt = alias_tables(inp.block_tables.cpu().numpy(), bs)

    def run(x):
        o = tq.decode_tq4(x.q, x.cache, x.centroids, x.block_tables, x.seq_lens, num_kv_heads=2,
                          kv_block_size=bs, num_partitions=4, softmax_scale=x.softmax_scale,
                          max_seq_len=max(LENS), fused=(path == "fused"))
        torch.cuda.synchronize()
        return o

    aliased = dataclasses.replace(inp, block_tables=torch.from_numpy(bt).cuda())
    say(f"[aliasing] 4-bit bs={bs} {path}")
    out = run(aliased)
    c = aliased.to("cpu")
    ref64 = oracle.decode_tq4(c.q, c.cache, c.centroids, c.block_tables, c.seq_lens,
                              inp.softmax_scale, 2, bs, nthreads=ORACLE_THREADS)
    compare(out, ref64, f"tq4 aliased bs{bs} {path}")
    bt2, extra = dealias(bt, bs, inp.num_blocks)
    src = torch.tensor(extra, dtype=torch.int64, device="cuda")
    flat = dataclasses.replace(inp, block_tables=torch.from_numpy(bt2).cuda(),
                               cache=torch.cat([inp.cache, inp.cache[src]]).contiguous(),
                               num_blocks=inp.num_blocks + len(extra))
    assert torch.equal(out.view(torch.int16), run(flat).view(torch.int16))
