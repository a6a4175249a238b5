"""Seeded random shapes through both cache formats and both paths, against the fp64 oracle
(bf16 out: max abs <= 1e-2, mean abs <= 1e-3).  Each case draws the batch size, kv heads,
query group, block size, tile groups per partition, a partition count at or above the one
the lengths need, and ragged lengths with empty sequences and block- and chunk-edge values,
so that the launch plans (per-partition or flat partition kernel, non-temporal partials or
not, even split or per-(s, h) workgroups) and the work-list boundaries fall in many places.
Needs an MI355X."""

import numpy as np
import pytest

import workloads
from gpu_util import PATHS, compare, gpu_decode, oracle_decode, say
from test_gpu_tq4 import gpu_tq4, oracle_tq4

pytestmark = pytest.mark.gpu

EDGES = (0, 1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513)


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    qg = int(rng.choice((6, 8, 16)))
    bs = int(rng.choice((16, 32)))
    G = int(rng.choice((1, 1, 2, 5)))
    hkv = int(rng.choice((1, 2, 4, 8)))
    S = int(rng.integers(1, max(2, 320 // hkv)))
    max_len = int(rng.choice((300, 1000, 2500)))
    lens = rng.integers(0, max_len + 1, size=S)
    k = min(S, len(EDGES) // 2)
    lens[:k] = rng.choice(EDGES, size=k)
    lens = tuple(int(x) for x in lens)
    need = max(1, -(-max(lens) // (256 * G)))
    P = need + int(rng.integers(0, 3))
    return dict(qg=qg, bs=bs, G=G, hkv=hkv, S=S, lens=lens, P=P, seed=2000 + i)


def big_case(i, qg, bs, G, hkv, S, max_len, P):
    """A larger batch whose plan crosses a size threshold (non-temporal partials; the flat
    partition kernel of the 4-bit format; a length scan past 256 sequences)."""
    rng = np.random.default_rng(3000 + i)
    lens = rng.integers(0, max_len + 1, size=S)
    lens[:4] = (max_len, 0, 1, 257)
    return dict(qg=qg, bs=bs, G=G, hkv=hkv, S=S, lens=tuple(int(x) for x in lens), P=P,
                seed=4000 + i)


CASES = [draw_case(i) for i in range(10)] + [
    big_case(0, 8, 16, 1, 8, 200, 2048, 8),   # fp8 partials >= 24 MiB (bound): non-temporal
    big_case(1, 16, 32, 1, 4, 300, 1024, 4),  # 4800 partitions: the 4-bit flat partition kernel
]


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_random_shapes(case, fmt):
    c = case
    wl = workloads.small_workload(name="rand", num_seqs=c["S"], num_kv_heads=c["hkv"],
                                  query_group_size=c["qg"], kv_block_size=c["bs"],
                                  seq_lens=c["lens"], tile_groups_per_partition=c["G"],
                                  seed=c["seed"])
    desc = (f"{fmt} S={c['S']} Hkv={c['hkv']} QG={c['qg']} BS={c['bs']} G={c['G']} P={c['P']} "
            f"max L={max(c['lens'])}")
    say(f"[random] {desc}")
    if fmt == "fp8":
        inp = workloads.make_inputs(wl, device="cuda", seq_lens=c["lens"], num_partitions=c["P"])
        ref = oracle_decode(inp)
        for path in PATHS:
            out = gpu_decode(inp, num_partitions=c["P"], tile_groups=c["G"], path=path)
            compare(out, ref, f"{desc} {path}")
    else:
        inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=c["lens"],
                                        num_partitions=c["P"])
        ref = oracle_tq4(inp)
        for path in PATHS:
            out = gpu_tq4(inp, path, num_partitions=c["P"], tile_groups=c["G"])
            compare(out, ref, f"{desc} {path}")
