"""HIP path vs the fp64 oracle, element by element (bf16 out: max abs <= 1e-2,
mean abs <= 1e-3).  Needs an MI355X."""

import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_util import PATHS, cached_ref, compare, gpu_decode, oracle_decode, say

pytestmark = pytest.mark.gpu

WORKLOADS = ["w1_tiny", "w2_s32_ctx4k", "w3_s64_ragged", "w4_s128_ctx8k", "w5_s16_long"]


@pytest.mark.parametrize("name", WORKLOADS)
@pytest.mark.parametrize("path", PATHS)
def test_workload_parity(path, name):
    """Every output element of each workload, both paths, against one oracle reference per
    workload (the bandwidth workload w4 included: 1024 (s, h) units x 8 rows x 128)."""
    wl = workloads.WORKLOADS[name]
    say(f"[parity] {name} {path}: generating on cuda:0")
    inp = workloads.make_inputs(wl, device="cuda")
    say(f"[parity] {name} {path}: S={wl.num_seqs} Hkv={wl.num_kv_heads} QG={wl.query_group_size} "
        f"BS={wl.kv_block_size} P={inp.num_partitions} G={wl.tile_groups_per_partition} "
        f"NB={inp.num_blocks} maxL={int(inp.seq_lens.max())}")
    out = gpu_decode(inp, path=path)
    ref = cached_ref(("fp8", name), lambda: oracle_decode(inp))
    compare(out, ref, f"{name} {path}")


SWEEP_LENS = (1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 300, 513, 1000)
SWEEP = [(qg, bs) for qg in (6, 8, 16) for bs in (16, 32)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("qg,bs", SWEEP, ids=[f"qg{q}_bs{b}" for q, b in SWEEP])
def test_small_sweep(qg, bs, path):
    lens = SWEEP_LENS
    wl = workloads.small_workload(name=f"sweep_qg{qg}_bs{bs}", num_seqs=len(lens), num_kv_heads=3,
                                  query_group_size=qg, kv_block_size=bs, seq_lens=lens,
                                  seed=100 + qg + bs)
    for G, P in ((1, 4), (1, 7), (2, 2), (3, 2), (5, 1)):
        say(f"[sweep] {path} qg={qg} bs={bs} G={G} P={P} lens={lens}")
        inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P)
        out = gpu_decode(inp, num_partitions=P, tile_groups=G, path=path)
        compare(out, oracle_decode(inp), f"{path} qg{qg} bs{bs} G{G} P{P}")


@pytest.mark.parametrize("path", PATHS)
def test_zero_lengths_and_outliers(path):
    lens = (0, 1, 700, 0, 33)
    wl = workloads.small_workload(name="zeros", num_seqs=len(lens), num_kv_heads=2,
                                  query_group_size=16, kv_block_size=32, seq_lens=lens, seed=7,
                                  outlier_frac=0.01)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=3)
    say(f"[zeros] {path}: lens with zeros, outlier q channels")
    out = gpu_decode(inp, num_partitions=3, tile_groups=1, path=path)
    assert (out[0].float() == 0).all() and (out[3].float() == 0).all()
    compare(out, oracle_decode(inp), f"{path} zero lengths + outliers")


def test_partials_match_oracle():
    """The partial triple itself (fp32) against the oracle's split-K partials."""
    import oracle
    import paged_gqa_decode_amd as tq

    lens = (40, 256, 257, 600)
    wl = workloads.small_workload(name="partials", num_seqs=4, num_kv_heads=2, query_group_size=8,
                                  kv_block_size=16, seq_lens=lens, seed=11)
    P, G = 3, 1
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P)
    part = tq.alloc_partials(4, 2, P, 8, "cuda")
    for t in (part.out, part.max_logits, part.exp_sums):
        t.fill_(float("nan"))
    say("[partials] P=3 G=1")
    gpu_decode(inp, num_partitions=P, tile_groups=G, partials=part)
    c = inp.to("cpu")
    o, m, l = oracle.partials(c.q, c.k_cache, c.v_cache, c.kv_scales, c.block_tables, c.seq_lens,
                              inp.softmax_scale, P, 256 * G)
    live = ~np.isnan(m)
    gm = part.max_logits.cpu().numpy()
    gl = part.exp_sums.cpu().numpy()
    go = part.out.cpu().numpy()
    assert np.array_equal(np.isnan(gm), ~live), "dead partitions must stay untouched"
    assert np.max(np.abs(gm[live] - m[live])) < 1e-4 * max(1.0, np.abs(m[live]).max())
    assert np.max(np.abs(gl[live] / l[live] - 1)) < 2e-3
    err = np.abs(go[live] - o[live]).max()
    say(f"  partial o max abs err {err:.3e}")
    assert err < 5e-3


def test_fused_split_modes():
    """tq_decode_fused with no workspace (one workgroup per (s, h)), the full workspace (the
    tokens of an (s, h) split over several workgroups, last arrival merges) and a workspace
    that fits only two workgroups per (s, h): all match the oracle; repeated calls give the
    same bits; the arrival counters are left at zero; garbage in the partial area is harmless."""
    import paged_gqa_decode_amd as tq

    lens = (5000, 37, 3000, 8191)
    wl = workloads.small_workload(name="splits", num_seqs=4, num_kv_heads=1, query_group_size=16,
                                  kv_block_size=32, seq_lens=lens, seed=17)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=32)
    ref = oracle_decode(inp)
    S, Hkv, QG, maxlen = 4, 1, 16, max(lens)
    full = tq.fused_workspace_bytes(S, Hkv, QG, maxlen)
    assert full > 0, "these sizes should split each (s, h) over several workgroups"

    def run(ws):
        out = torch.empty((S, Hkv * QG, 128), dtype=torch.bfloat16, device="cuda")
        tq.tq_decode_fused(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables,
                           inp.seq_lens, out, Hkv, QG, 32, 1, inp.softmax_scale, num_partitions=32,
                           max_seq_len=maxlen, workspace=ws)
        torch.cuda.synchronize()
        return out

    say("[splits] no workspace")
    a = run(None)
    compare(a, ref, "fused, one workgroup per (s, h)")
    ws = torch.zeros(full, dtype=torch.uint8, device="cuda")
    ws[256:] = 0xFF  # NaN garbage in the partial area; the counters (first 256 B) stay zero
    say(f"[splits] full workspace ({full} B)")
    b1 = run(ws)
    compare(b1, ref, "fused, split over workgroups")
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "counters must be re-armed to 0"
    b2 = run(ws)
    assert torch.equal(b1.view(torch.int16), b2.view(torch.int16))
    # a workspace with room for exactly two workgroups per (s, h)
    rows = S * Hkv * 2 * QG
    two = 256 + ((rows * 512 + 255) // 256) * 256 + 2 * ((rows * 4 + 255) // 256) * 256
    ws2 = torch.zeros(two, dtype=torch.uint8, device="cuda")
    say(f"[splits] two-split workspace ({two} B)")
    c = run(ws2)
    compare(c, ref, "fused, two workgroups per (s, h)")
    assert int(ws2[:256].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("path", PATHS)
def test_long_ranges_and_many_partitions(path):
    """A partition (or wave range) of more than 64 cache blocks, so the block-table window is
    reloaded mid-stream (G=8, BS=16: 128 blocks per partition), and a merge over more than
    256 live partitions (G=1, 280 partitions), which takes the merge kernel's unstaged path."""
    lens = (1500, 2048, 700, 4096)
    wl = workloads.small_workload(name="longrange", num_seqs=4, num_kv_heads=2, query_group_size=8,
                                  kv_block_size=16, seq_lens=lens, seed=23)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=2)
    say(f"[longrange] {path} G=8 P=2 BS=16")
    out = gpu_decode(inp, num_partitions=2, tile_groups=8, path=path)
    compare(out, oracle_decode(inp), f"{path} G8 BS16 (window reload)")
    lens = (280 * 256 - 5, 3000)
    wl = workloads.small_workload(name="manyparts", num_seqs=2, num_kv_heads=1, query_group_size=6,
                                  kv_block_size=32, seq_lens=lens, seed=29)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=280)
    say(f"[manyparts] {path} G=1 P=280 L={lens}")
    out = gpu_decode(inp, num_partitions=280, tile_groups=1, path=path)
    compare(out, oracle_decode(inp), f"{path} 280 partitions")


def _fused_vs_oracle(inp, S, Hkv, QG, BS, maxlen, P, ws_bytes=None, what=""):
    import paged_gqa_decode_amd as tq

    nbytes = tq.fused_workspace_bytes(S, Hkv, QG, maxlen) if ws_bytes is None else ws_bytes
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda") if nbytes else None
    out = torch.full((S, Hkv * QG, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    tq.tq_decode_fused(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables,
                       inp.seq_lens, out, Hkv, QG, BS, 1, inp.softmax_scale, num_partitions=P,
                       max_seq_len=maxlen, workspace=ws)
    torch.cuda.synchronize()
    compare(out, oracle_decode(inp), what)
    if ws is not None:
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "counters must be re-armed"
    return out


def test_even_split_one_long_sequence():
    """One (s, h) of 1280 32-token entries: one wave per entry, 160 workgroups, and a merge of
    160 workgroup partials (more than the merge keeps in registers)."""
    lens = (40960,)
    wl = workloads.small_workload(name="onelong", num_seqs=1, num_kv_heads=1, query_group_size=16,
                                  kv_block_size=32, seq_lens=lens, seed=41)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=160)
    say("[even] one sequence of 40960 tokens, QG 16")
    _fused_vs_oracle(inp, 1, 1, 16, 32, 40960, 160, what="fused, one long sequence")


def test_even_split_ragged_with_empty_sequences():
    """Lengths around tile-group edges, empty sequences between live ones, three kv heads: the
    even split cuts (s, h) ranges at every kind of boundary."""
    rng = np.random.default_rng(43)
    base = [0, 1, 255, 256, 257, 511, 1000, 5000, 0, 3000]
    lens = tuple(int(x) for x in rng.permutation(base * 4))
    wl = workloads.small_workload(name="evenrag", num_seqs=len(lens), num_kv_heads=3,
                                  query_group_size=6, kv_block_size=16, seq_lens=lens, seed=44)
    maxlen = max(lens)
    P = (maxlen + 255) // 256
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P)
    say(f"[even] ragged with empty sequences: S={len(lens)} Hkv=3 QG=6 BS=16")
    out = _fused_vs_oracle(inp, len(lens), 3, 6, 16, maxlen, P, what="fused, ragged + empty")
    for s, L in enumerate(lens):
        if L == 0:
            assert (out[s].float() == 0).all()


@pytest.mark.parametrize("S", [1024, 1025])
def test_even_split_sequence_limit(S):
    """1024 sequences take the even split, 1025 the per-(s, h) workgroups; both match the oracle."""
    rng = np.random.default_rng(45 + S)
    lens = tuple(int(x) for x in rng.integers(1, 700, size=S))
    wl = workloads.small_workload(name=f"lim{S}", num_seqs=S, num_kv_heads=1, query_group_size=8,
                                  kv_block_size=32, seq_lens=lens, seed=46)
    maxlen = max(lens)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=3)
    say(f"[even] S={S}")
    _fused_vs_oracle(inp, S, 1, 8, 32, maxlen, 3, what=f"fused, S={S}")


@pytest.mark.parametrize("path", PATHS)
def test_signed_scales(path):
    """K and V scales of either sign (the format reads code * scale, nothing makes a scale
    non-negative): a random half of them negated, and a batch whose V scales are all negative,
    against the oracle."""
    lens = (1, 40, 333, 1000)
    wl = workloads.small_workload(name="signed", num_seqs=len(lens), num_kv_heads=2,
                                  query_group_size=8, kv_block_size=16, seq_lens=lens, seed=47)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=4)
    g = torch.Generator(device="cuda").manual_seed(48)
    flip = torch.where(torch.rand(inp.kv_scales.shape, generator=g, device="cuda") < 0.5, -1.0, 1.0)
    mixed = dataclasses.replace(inp, kv_scales=inp.kv_scales * flip)
    say(f"[signed scales] {path}: half of the K and V scales negated")
    compare(gpu_decode(mixed, path=path), oracle_decode(mixed), f"{path} mixed-sign scales")
    sc = inp.kv_scales.clone()
    sc[:, :, 1, :] = -sc[:, :, 1, :]
    neg = dataclasses.replace(inp, kv_scales=sc)
    say(f"[signed scales] {path}: every V scale negative")
    out = gpu_decode(neg, path=path)
    compare(out, oracle_decode(neg), f"{path} negative V scales")
    # negating every V scale negates the output exactly
    assert torch.equal(out.float(), -gpu_decode(inp, path=path).float())
