"""The 4-bit record format on the GPU against the fp64 oracle (bf16 out: max abs <= 1e-2, mean
abs <= 1e-3), both paths (tq4_decode + tq_decode_reduce, and tq4_decode_fused), and its
bit-exact properties.  Needs an MI355X."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_amd as tq
import workloads
from gpu_util import ORACLE_THREADS, PATHS, cached_ref, compare, say

pytestmark = pytest.mark.gpu


def gpu_tq4(inp, path, num_partitions=None, tile_groups=None):
    wl = inp.wl
    G = wl.tile_groups_per_partition if tile_groups is None else tile_groups
    P = inp.num_partitions if num_partitions is None else num_partitions
    out = tq.decode_tq4(inp.q, inp.cache, inp.centroids, inp.block_tables, inp.seq_lens,
                        num_kv_heads=wl.num_kv_heads, kv_block_size=wl.kv_block_size,
                        num_partitions=P, tile_groups_per_partition=G,
                        softmax_scale=inp.softmax_scale,
                        max_seq_len=int(inp.seq_lens.max().item()), fused=(path == "fused"),
                        kv_layout=inp.kv_layout)
    torch.cuda.synchronize()
    return out


def oracle_tq4(inp, units=None):
    c = inp.to("cpu")
    return oracle.decode_tq4(c.q, c.cache, c.centroids, c.block_tables, c.seq_lens,
                             inp.softmax_scale, inp.wl.num_kv_heads, inp.wl.kv_block_size,
                             units=units, nthreads=ORACLE_THREADS, layout=inp.kv_layout)


def bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


SWEEP_LENS = (1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 300, 513, 1000)
SWEEP = [(qg, bs) for qg in (6, 8, 16) for bs in (16, 32)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("qg,bs", SWEEP, ids=[f"qg{q}_bs{b}" for q, b in SWEEP])
def test_tq4_small_sweep(qg, bs, path):
    lens = SWEEP_LENS
    wl = workloads.small_workload(name=f"tq4_qg{qg}_bs{bs}", num_seqs=len(lens), num_kv_heads=3,
                                  query_group_size=qg, kv_block_size=bs, seq_lens=lens,
                                  seed=200 + qg + bs)
    for G, P in ((1, 4), (2, 2), (5, 1)):
        say(f"[tq4 sweep] {path} qg={qg} bs={bs} G={G} P={P}")
        inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens, num_partitions=P)
        out = gpu_tq4(inp, path, num_partitions=P, tile_groups=G)
        compare(out, oracle_tq4(inp), f"tq4 {path} qg{qg} bs{bs} G{G} P{P}")


WORKLOADS = ["w2_s32_ctx4k", "w3_s64_ragged", "w4_s128_ctx8k", "w5_s16_long"]


@pytest.mark.parametrize("name", WORKLOADS)
@pytest.mark.parametrize("path", PATHS)
def test_tq4_workload_parity(path, name):
    """Every output element of each workload in the 4-bit format, both paths, against one
    oracle reference per workload (w4: 1024 (s, h) units x 8 rows x 128)."""
    wl = workloads.WORKLOADS[name]
    say(f"[tq4 parity] {name} {path}: generating")
    inp = workloads.make_inputs_tq4(wl, device="cuda")
    out = gpu_tq4(inp, path)
    ref = cached_ref(("tq4", name), lambda: oracle_tq4(inp))
    compare(out, ref, f"tq4 {name} {path}")


@pytest.mark.parametrize("path", PATHS)
def test_tq4_bandwidth_workload_repeat_runs(path):
    """The bandwidth workload (32 partitions per (s, h) on the two-kernel path, the even split
    over 2048 waves on the fused one) decoded three times: the same bits each time."""
    inp = workloads.make_inputs_tq4(workloads.WORKLOADS["w4_s128_ctx8k"], device="cuda")
    say(f"[tq4 bitwise] w4 three times, {path}")
    first = bits(gpu_tq4(inp, path))
    for _ in range(2):
        assert np.array_equal(bits(gpu_tq4(inp, path)), first)


@pytest.mark.parametrize("path", PATHS)
def test_tq4_signed_metadata(path):
    """fp16 K norms and V scales of either sign, against the oracle: the K norm's sign bit set
    on a random half of the rows, and on another random half of the rows both the V scale and
    the V zero point negated (which negates those V rows exactly, so the output keeps the
    magnitude for which bf16's own rounding stays inside the bound).  Negating the V scale and
    zero point of every row negates V: that output matches the oracle too.  (Unlike the fp8
    path's, it is not required to be the exact negation of the original output: the 4-bit PV
    product runs on index bytes offset by 1024 in f16, and the offset is taken out after the
    MFMA's fp32 accumulation, whose rounding need not be symmetric under a sign change.)"""
    inp = _small((1, 40, 333, 1000), qg=16, bs=32, P=4, seed=63)
    Hkv, BS = inp.wl.num_kv_heads, inp.wl.kv_block_size
    data_bytes = Hkv * BS * 128
    meta = inp.cache[:, data_bytes:].contiguous().view(torch.int16).view(-1, Hkv, 3, BS)
    g = torch.Generator(device="cuda").manual_seed(64)

    def with_meta(m):
        c = inp.cache.clone()
        c[:, data_bytes:] = m.contiguous().view(torch.uint8).view(c.shape[0], -1)
        return dataclasses.replace(inp, cache=c)

    sign = torch.tensor(-32768, dtype=torch.int16, device="cuda")  # the fp16 sign bit
    k_flip = torch.rand(meta[:, :, 0].shape, generator=g, device="cuda") < 0.5
    v_flip = torch.rand(meta[:, :, 0].shape, generator=g, device="cuda") < 0.5
    mixed = meta.clone()
    mixed[:, :, 0] = torch.where(k_flip, mixed[:, :, 0] ^ sign, mixed[:, :, 0])
    for f in (1, 2):
        mixed[:, :, f] = torch.where(v_flip, mixed[:, :, f] ^ sign, mixed[:, :, f])
    assert (mixed[:, :, 1] < 0).any() and (mixed[:, :, 1] > 0).any()
    x = with_meta(mixed)
    say(f"[tq4 signed metadata] {path}: mixed-sign K norms and V scales")
    compare(gpu_tq4(x, path), oracle_tq4(x), f"tq4 {path} mixed-sign metadata")
    neg = meta.clone()
    neg[:, :, 1:] ^= sign  # every V scale and zero point negated
    x = with_meta(neg)
    out = gpu_tq4(x, path)
    compare(out, oracle_tq4(x), f"tq4 {path} negative V scales")
    diff = (out.float() + gpu_tq4(inp, path).float()).abs().max().item()
    say(f"  max |out(-V) + out(V)| = {diff:.3e}")


def _small(lens, qg=8, bs=16, hkv=2, seed=5, P=None):
    wl = workloads.small_workload(name="tq4bit", num_seqs=len(lens), num_kv_heads=hkv,
                                  query_group_size=qg, kv_block_size=bs, seq_lens=lens, seed=seed)
    return workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens, num_partitions=P)


@pytest.mark.parametrize("path", PATHS)
def test_tq4_determinism_relabelling_and_poison(path):
    """Same bits run to run; relabelling physical blocks (with a consistent table) and
    garbage past the lengths (random index bytes, NaN metadata, garbage table tails) change
    nothing."""
    inp = _small((1, 40, 333, 1000), bs=32, P=4, seed=21)
    say(f"[tq4 bitwise] {path}")
    ref = gpu_tq4(inp, path)
    assert np.array_equal(bits(gpu_tq4(inp, path)), bits(ref))
    NB = inp.num_blocks
    perm = torch.from_numpy(np.random.default_rng(3).permutation(NB).astype(np.int64)).cuda()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(NB, device="cuda")
    moved = dataclasses.replace(inp, cache=inp.cache[inv].contiguous(),
                                block_tables=perm[inp.block_tables.long()].to(torch.int32))
    assert np.array_equal(bits(gpu_tq4(moved, path)), bits(ref))
    assert np.array_equal(bits(gpu_tq4(workloads.poison_tq4(inp), path)), bits(ref))


@pytest.mark.parametrize("qg,bs", [(8, 16), (16, 32), (6, 32)])
def test_tq4_single_tile_group_identity(qg, bs):
    """L <= 256: every (P, G) choice gives the same bits on each path; across the paths, the
    sequences of at most one 32-token entry of the fused path's work list agree too."""
    lens = (1, 16, 31, 100, 255, 256)
    inp = _small(lens, qg=qg, bs=bs, P=1, seed=30 + qg)
    say(f"[tq4 identity] qg={qg} bs={bs}")
    first = {}
    for path in PATHS:
        for P, G in ((1, 1), (3, 1), (1, 5), (2, 2)):
            o = bits(gpu_tq4(inp, path, num_partitions=P, tile_groups=G))
            first.setdefault(path, o)
            assert np.array_equal(o, first[path]), (path, P, G)
    whole = [i for i, L in enumerate(lens) if L <= 32]
    a, b = (first[p] for p in PATHS)
    assert np.array_equal(a[whole], b[whole])


# Batches whose partitions (bounded by the longest length) fill the device's resident round
# of 2048 waves take the flat partition kernel for the 4-bit format; smaller ones (here each
# sequence decoded alone) take one wave per partition.  The last case fills exactly one round.
FLAT_CASES = [(8, 32, 1, 64, 4, 4096), (16, 16, 2, 48, 8, 6000), (6, 32, 5, 128, 8, 6400),
              (8, 16, 1, 600, 2, 1024), (16, 32, 1, 64, 4, 2048)]


@pytest.mark.parametrize("qg,bs,G,S,hkv,max_len", FLAT_CASES,
                         ids=[f"qg{c[0]}_bs{c[1]}_G{c[2]}" for c in FLAT_CASES])
def test_tq4_flat_partition_kernel(qg, bs, G, S, hkv, max_len):
    """The batch's partials (flat partition kernel) equal bit for bit those of the same
    sequences decoded one at a time (one wave per partition), written entries and untouched
    ones alike; the merged batch matches the oracle."""
    E = 256 * G
    rng = np.random.default_rng(70 + qg + G)
    lens = rng.integers(0, max_len + 1, size=S)
    lens[:6] = (max_len, 0, 1, E - 1, E, E + 1)
    lens = tuple(int(x) for x in lens)
    P = -(-max_len // E)
    assert S * hkv * P >= 2048 and hkv * P < 2048
    wl = workloads.small_workload(name="tq4flat", num_seqs=S, num_kv_heads=hkv, query_group_size=qg,
                                  kv_block_size=bs, seq_lens=lens, tile_groups_per_partition=G,
                                  seed=80 + qg)
    inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens, num_partitions=P)
    say(f"[tq4 flat partition] qg={qg} bs={bs} G={G} S={S} Hkv={hkv} P={P}")

    def partials(sl):
        n = sl.stop - sl.start
        part = tq.alloc_partials(n, hkv, P, qg, "cuda")
        for t in (part.out, part.max_logits, part.exp_sums):
            t.fill_(float("nan"))
        tq.tq4_decode(inp.q[sl].contiguous(), inp.cache, inp.centroids,
                      inp.block_tables[sl].contiguous(), inp.seq_lens[sl].contiguous(), part, hkv,
                      qg, bs, G, inp.softmax_scale, num_partitions=P, max_seq_len=max_len)
        torch.cuda.synchronize()
        return part

    whole = partials(slice(0, S))
    for s in (0, 1, 2, 3, 4, 5, S // 2, S - 1):
        one = partials(slice(s, s + 1))
        for a, b in ((whole.out, one.out), (whole.max_logits, one.max_logits),
                     (whole.exp_sums, one.exp_sums)):
            assert torch.equal(a[s:s + 1].view(torch.int32), b.view(torch.int32)), (s, lens[s])
    out = torch.empty((S, hkv * qg, 128), dtype=torch.bfloat16, device="cuda")
    tq.tq_decode_reduce(whole, inp.seq_lens, out, hkv, qg, G, num_partitions=P, max_seq_len=max_len)
    torch.cuda.synchronize()
    compare(out, oracle_tq4(inp), f"tq4 flat partition qg{qg} bs{bs} G{G}")


@pytest.mark.parametrize("path", PATHS)
def test_tq4_query_power_of_two_scaling(path):
    """The query enters the 4-bit path's MFMA in f16.  q * 2^k with softmax_scale * 2^-k has
    the same logits: the output is the same bits, for k = 8 (|q| stays below 2^15) and k = 16
    (|q| passes 2^15, and the kernel scales q down by a power of two before the conversion).
    Elements of q below 2^-10 are zeroed first, so no value becomes an f16 subnormal."""
    inp = _small((1, 77, 300, 700), qg=8, bs=32, P=3, seed=61)
    q = inp.q.float()
    q = torch.where(q.abs() < 2.0 ** -10, torch.zeros_like(q), q).to(torch.bfloat16)
    base = dataclasses.replace(inp, q=q)
    say(f"[tq4 q scaling] {path}, max |q| {q.float().abs().max().item():.2f}")
    ref = gpu_tq4(base, path)
    for k in (8, 16):
        scaled = dataclasses.replace(base, q=(q.float() * 2.0 ** k).to(torch.bfloat16),
                                     softmax_scale=base.softmax_scale * 2.0 ** -k)
        assert float(scaled.q.float().abs().max()) >= (2.0 ** 15 if k == 16 else 0.0)
        assert np.array_equal(bits(gpu_tq4(scaled, path)), bits(ref)), k


def test_tq4_fused_workspace_modes():
    """tq4_decode_fused with no workspace (one workgroup per (s, h)), with room for exactly two
    workgroups per (s, h) (the per-(s, h) plan split in two, merged by the last arrival), and
    with the full workspace (the even split over the whole batch): all match the oracle, and
    the arrival counters are left at zero."""
    lens = (5000, 37, 3000, 8191)
    S, Hkv, QG, BS, P = 4, 1, 16, 32, 32
    wl = workloads.small_workload(name="tq4ws", num_seqs=S, num_kv_heads=Hkv, query_group_size=QG,
                                  kv_block_size=BS, seq_lens=lens, seed=19)
    inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens, num_partitions=P)
    ref = oracle_tq4(inp)
    maxlen = max(lens)
    rows = S * Hkv * 2 * QG
    two = 256 + ((rows * 512 + 255) // 256) * 256 + 2 * ((rows * 4 + 255) // 256) * 256
    full = tq.fused_workspace_bytes(S, Hkv, QG, maxlen)
    assert full > two
    for what, nbytes in (("no workspace", 0), ("two workgroups per (s, h)", two),
                         ("full workspace", full)):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
        out = torch.empty((S, Hkv * QG, 128), dtype=torch.bfloat16, device="cuda")
        say(f"[tq4 workspace] {what}")
        tq.tq4_decode_fused(inp.q, inp.cache, inp.centroids, inp.block_tables, inp.seq_lens, out,
                            Hkv, QG, BS, 1, inp.softmax_scale, num_partitions=P, max_seq_len=maxlen,
                            workspace=ws)
        torch.cuda.synchronize()
        compare(out, ref, f"tq4 fused, {what}")
        if ws is not None:
            assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "counters must be re-armed"
