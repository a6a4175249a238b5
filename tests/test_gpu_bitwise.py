"""Bit-exact properties of the HIP path (needs an MI355X):
run-to-run determinism, block-table indexing (physical block relabelling and
a one-hot gather probe), the single-live-partition identity across partition
counts and tile groups, poison invariance, and V-magnitude equivariance."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_gqa_decode_amd as tq
import workloads
from gpu_util import PATHS, gpu_decode, say

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


def small(lens, qg=8, bs=16, hkv=2, seed=5, P=None):
    wl = workloads.small_workload(name="bitwise", num_seqs=len(lens), num_kv_heads=hkv,
                                  query_group_size=qg, kv_block_size=bs, seq_lens=lens, seed=seed)
    return workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", ["w2_s32_ctx4k", "w3_s64_ragged", "w4_s128_ctx8k"])
def test_run_to_run_determinism(path, name):
    """The same bits on repeated runs; on the bandwidth workload (32 partitions per (s, h), 1024
    (s, h)), three runs, so that a read of partials or staged V before they are complete
    would show as a difference."""
    inp = workloads.make_inputs(workloads.WORKLOADS[name], device="cuda")
    reps = 3 if name == "w4_s128_ctx8k" else 2
    say(f"[bitwise] {name} {reps} times, {path}")
    first = bits(gpu_decode(inp, path=path))
    for _ in range(reps - 1):
        assert np.array_equal(bits(gpu_decode(inp, path=path)), first)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [16, 32])
def test_block_relabelling_is_invisible(bs, path):
    inp = small((1, 40, 333, 1000), bs=bs, P=4, seed=21)
    say(f"[bitwise] block relabelling bs={bs} {path}")
    ref = gpu_decode(inp, path=path)
    NB = inp.num_blocks
    perm = torch.from_numpy(np.random.default_rng(3).permutation(NB).astype(np.int64)).cuda()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(NB, device="cuda")
    moved = dataclasses.replace(
        inp, k_cache=inp.k_cache[inv].contiguous(), v_cache=inp.v_cache[inv].contiguous(),
        kv_scales=inp.kv_scales[inv].contiguous(),
        block_tables=perm[inp.block_tables.long()].to(torch.int32))
    assert np.array_equal(bits(gpu_decode(moved, path=path)), bits(ref))


@pytest.mark.parametrize("qg,bs", [(8, 16), (16, 32), (6, 32)])
def test_single_live_partition_identity(qg, bs):
    """L <= 256: (P=1, G=1), (P=3, G=1), (P=1, G=5), (P=2, G=2) give the same bits on each
    path.  Across the paths the bits agree for the sequences the fused path does not split
    (L <= 32, one entry of its work list); longer ones it may split between waves."""
    lens = (1, 16, 31, 100, 255, 256)
    inp = small(lens, qg=qg, bs=bs, P=1, seed=30 + qg)
    first = {}
    for path in PATHS:
        for P, G in ((1, 1), (3, 1), (1, 5), (2, 2)):
            say(f"[bitwise] single live partition qg={qg} bs={bs} P={P} G={G} {path}")
            o = bits(gpu_decode(inp, num_partitions=P, tile_groups=G, path=path))
            first.setdefault(path, o)
            assert np.array_equal(o, first[path]), (path, P, G)
    whole = [i for i, L in enumerate(lens) if L <= 32]
    a, b = (first[p] for p in PATHS)
    assert np.array_equal(a[whole], b[whole])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [16, 32])
def test_poison_invariance(bs, path):
    """Garbage past each sequence end, in unused table entries and in the partial buffers."""
    lens = (1, 17, 250, 333, 769)
    inp = small(lens, bs=bs, P=4, seed=40)
    say(f"[bitwise] poison bs={bs} {path}")
    clean = gpu_decode(inp, path=path)
    dirty = workloads.poison(inp)
    part = tq.alloc_partials(len(lens), 2, 4, 8, "cuda")
    for t in (part.out, part.max_logits, part.exp_sums):
        t.fill_(float("nan"))
    out = torch.full_like(clean, float("nan"))
    got = gpu_decode(dirty, partials=part, out=out, path=path)
    assert np.array_equal(bits(got), bits(clean))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs,P", [(16, 1), (32, 3)])
def test_one_hot_gather_probe(bs, P, path):
    """K is zero except at token t*, whose logit leads by ~724, so every other weight is exactly
    0 in fp32: out == bf16(V[t*]) bit for bit."""
    L = 200 if P == 1 else 700
    inp = small((L, L), qg=8, bs=bs, P=P, seed=50)
    Hkv, QG = 2, 8
    rng = np.random.default_rng(51)
    sc = inp.kv_scales.clone()
    sc[:, :, 1, :] = torch.from_numpy(
        2.0 ** rng.integers(-8, 1, size=tuple(sc[:, :, 1, :].shape))).float().cuda()
    sc[:, :, 0, :] = 1.0
    q = torch.ones_like(inp.q)
    bt = inp.block_tables.cpu().numpy()
    v64 = (inp.v_cache.view(torch.float8_e4m3fn).double() *
           sc[:, :, 1, :].unsqueeze(-1).double())  # [NB][Hkv][BS][D]
    sweep = [0, 1, bs - 1, bs, bs + 1, 2 * bs - 1, 100, L - 1] + ([255, 256, 257, 511, 512] if P > 1 else [])
    for tstar in sweep:
        k = torch.zeros_like(inp.k_cache)
        sck = sc.clone()
        for s in range(2):
            blk, slot = int(bt[s, tstar // bs]), tstar % bs
            k[blk, :, slot] = 0x38  # 1.0
            sck[blk, :, 0, slot] = 64.0  # logit 128 * 64 / sqrt(128) ~ 724
        probe = dataclasses.replace(inp, q=q, k_cache=k, kv_scales=sck)
        say(f"[bitwise] one-hot probe bs={bs} P={P} t*={tstar} {path}")
        out = gpu_decode(probe, path=path)
        for s in range(2):
            blk, slot = int(bt[s, tstar // bs]), tstar % bs
            for h in range(Hkv):
                want = v64[blk, h, slot].float().to(torch.bfloat16)  # exact: code * 2^k
                assert torch.equal(want.float(), v64[blk, h, slot].float())
                for g in range(QG):
                    # value equality: a zero component may come out as +0 where V holds -0
                    assert torch.equal(out[s, h * QG + g].float(), want.float()), (tstar, s, h, g)


@pytest.mark.parametrize("path", PATHS)
def test_v_magnitude_equivariance(path):
    """Scaling every V scale by 2^20 (or 2^-20) scales the output by exactly that."""
    inp = small((5, 300, 1000), qg=16, bs=32, P=4, seed=60)
    say(f"[bitwise] V magnitude equivariance {path}")
    ref = gpu_decode(inp, path=path).float()
    for e in (20, -20):
        sc = inp.kv_scales.clone()
        sc[:, :, 1, :] *= 2.0 ** e
        got = gpu_decode(dataclasses.replace(inp, kv_scales=sc), path=path).float()
        assert torch.equal(got, ref * 2.0 ** e)


def test_partials_independent_of_batch_and_store_policy():
    """A batch with 24 MiB or more of fp8 partials (bound S * Hkv * P * QG * 520 B) stores
    them with the non-temporal bit; one sequence alone stores them plainly.  The partials of
    each sequence are the same bits either way, written entries and untouched ones alike."""
    S, hkv, qg, bs, P = 64, 8, 8, 16, 16
    assert S * hkv * P * qg * 520 >= 24 << 20 and hkv * P * qg * 520 < 24 << 20
    rng = np.random.default_rng(44)
    lens = rng.integers(0, 256 * P + 1, size=S)
    lens[:5] = (256 * P, 0, 1, 255, 257)
    lens = tuple(int(x) for x in lens)
    wl = workloads.small_workload(name="ntpartials", num_seqs=S, num_kv_heads=hkv,
                                  query_group_size=qg, kv_block_size=bs, seq_lens=lens, seed=45)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P)
    say(f"[bitwise] partials of a {S}-sequence batch against one sequence at a time")

    def partials(sl):
        part = tq.alloc_partials(sl.stop - sl.start, hkv, P, qg, "cuda")
        for t in (part.out, part.max_logits, part.exp_sums):
            t.fill_(float("nan"))
        tq.tq_decode(inp.q[sl].contiguous(), inp.k_cache, inp.v_cache, inp.kv_scales,
                     inp.block_tables[sl].contiguous(), inp.seq_lens[sl].contiguous(), part, hkv,
                     qg, bs, 1, inp.softmax_scale, num_partitions=P, max_seq_len=256 * P)
        torch.cuda.synchronize()
        return part

    whole = partials(slice(0, S))
    for s in (0, 1, 2, 3, 4, S // 2, S - 1):
        one = partials(slice(s, s + 1))
        for a, b in ((whole.out, one.out), (whole.max_logits, one.max_logits),
                     (whole.exp_sums, one.exp_sums)):
            assert torch.equal(a[s:s + 1].view(torch.int32), b.view(torch.int32)), (s, lens[s])
