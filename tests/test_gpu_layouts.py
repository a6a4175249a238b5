"""The page's slot-major row order at the boundary (ext->kv_layout = TQ_KV_LAYOUT_SLOT_MAJOR):
fp8 caches [NB][BS][Hkv][128] and 4-bit records whose data region is [BS][Hkv][128], as the
page's STEP F addresses them.  Both formats, both paths: against the oracle in that layout, and
bit for bit against the head-major decode of the same values (only the addresses differ, so
every kernel must produce the same bits).  The writer into a slot-major cache, bit for bit
against the oracle's writer.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_amd as tq
import workloads
from gpu_util import PATHS, cached_ref, compare, gpu_decode, oracle_decode, say
from test_gpu_tq4 import bits, gpu_tq4, oracle_tq4

pytestmark = pytest.mark.gpu

SWEEP_LENS = (1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 300, 513, 1000)
SWEEP = [(qg, bs) for qg in (6, 8, 16) for bs in (16, 32)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("qg,bs", SWEEP, ids=[f"qg{q}_bs{b}" for q, b in SWEEP])
def test_fp8_slot_major_sweep(qg, bs, path):
    wl = workloads.small_workload(name=f"slot_qg{qg}_bs{bs}", num_seqs=len(SWEEP_LENS),
                                  num_kv_heads=3, query_group_size=qg, kv_block_size=bs,
                                  seq_lens=SWEEP_LENS, seed=300 + qg + bs)
    for G, P in ((1, 4), (2, 2), (5, 1)):
        say(f"[slot-major] fp8 {path} qg={qg} bs={bs} G={G} P={P}")
        head = workloads.make_inputs(wl, device="cuda", seq_lens=SWEEP_LENS, num_partitions=P)
        slot = head.with_layout("slot")
        out = gpu_decode(slot, num_partitions=P, tile_groups=G, path=path)
        compare(out, oracle_decode(slot), f"fp8 slot-major {path} qg{qg} bs{bs} G{G} P{P}")
        ref = gpu_decode(head, num_partitions=P, tile_groups=G, path=path)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("qg,bs", SWEEP, ids=[f"qg{q}_bs{b}" for q, b in SWEEP])
def test_tq4_slot_major_sweep(qg, bs, path):
    wl = workloads.small_workload(name=f"slot4_qg{qg}_bs{bs}", num_seqs=len(SWEEP_LENS),
                                  num_kv_heads=3, query_group_size=qg, kv_block_size=bs,
                                  seq_lens=SWEEP_LENS, seed=400 + qg + bs)
    for G, P in ((1, 4), (5, 1)):
        say(f"[slot-major] 4-bit {path} qg={qg} bs={bs} G={G} P={P}")
        head = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=SWEEP_LENS, num_partitions=P)
        slot = head.with_layout("slot")
        out = gpu_tq4(slot, path, num_partitions=P, tile_groups=G)
        compare(out, oracle_tq4(slot), f"4-bit slot-major {path} qg{qg} bs{bs} G{G} P{P}")
        assert np.array_equal(bits(out), bits(gpu_tq4(head, path, num_partitions=P, tile_groups=G)))


WORKLOADS = ["w2_s32_ctx4k", "w3_s64_ragged", "w4_s128_ctx8k", "w5_s16_long"]


@pytest.mark.parametrize("name", WORKLOADS)
@pytest.mark.parametrize("path", PATHS)
def test_slot_major_workloads(path, name):
    """Each workload in the slot-major layout, both formats: the same bits as head-major, whose
    every output element is compared with the oracle in test_gpu_parity / test_gpu_tq4; the
    bandwidth workload w4 is also compared with the oracle in this layout directly."""
    wl = workloads.WORKLOADS[name]
    say(f"[slot-major] {name} {path}: fp8")
    head = workloads.make_inputs(wl, device="cuda")
    ref = gpu_decode(head, path=path)
    slot = head.with_layout("slot")
    del head
    out = gpu_decode(slot, path=path)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    if name == "w4_s128_ctx8k":
        compare(out, cached_ref(("fp8-slot", name), lambda: oracle_decode(slot)),
                f"fp8 slot-major {name} {path}")
    del slot, out, ref
    say(f"[slot-major] {name} {path}: 4-bit")
    head = workloads.make_inputs_tq4(wl, device="cuda")
    ref = gpu_tq4(head, path)
    slot = head.with_layout("slot")
    del head
    out = gpu_tq4(slot, path)
    assert np.array_equal(bits(out), bits(ref))
    if name == "w4_s128_ctx8k":
        compare(out, cached_ref(("tq4-slot", name), lambda: oracle_tq4(slot)),
                f"4-bit slot-major {name} {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [16, 32])
def test_slot_major_poison(bs, path):
    """Garbage past each sequence end (NaN codes and scales, random index bytes, NaN metadata)
    and in unused table entries, in the slot-major layout: the same bits as the clean cache."""
    lens = (1, 17, 250, 333, 769)
    wl = workloads.small_workload(name="slotpoison", num_seqs=len(lens), num_kv_heads=2,
                                  query_group_size=8, kv_block_size=bs, seq_lens=lens, seed=90 + bs)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=4, kv_layout="slot")
    say(f"[slot-major] poison bs={bs} {path}")
    clean = gpu_decode(inp, path=path)
    assert torch.equal(gpu_decode(workloads.poison(inp), path=path).view(torch.int16),
                       clean.view(torch.int16))
    inp4 = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens, num_partitions=4,
                                     kv_layout="slot")
    clean4 = gpu_tq4(inp4, path)
    assert np.array_equal(bits(gpu_tq4(workloads.poison_tq4(inp4), path)), bits(clean4))


@pytest.mark.parametrize("bs", [16, 32])
def test_slot_major_writer(bs):
    """tq_kv_write into a slot-major cache: codes and scales bit for bit against the oracle's
    writer in that layout, and the transposition of what it writes into a head-major cache."""
    from test_gpu_kv_write import make_rows

    T, Hkv, NB = 300, 4, 64
    rows = make_rows(T, Hkv, seed=50 + bs)
    rng = np.random.default_rng(60 + bs)
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    slots[::13] = -1
    kc = torch.from_numpy(rng.integers(0, 256, size=(NB, bs, Hkv, 128), dtype=np.uint8))
    vc = torch.from_numpy(rng.integers(0, 256, size=(NB, bs, Hkv, 128), dtype=np.uint8))
    sc = torch.from_numpy(rng.uniform(1, 2, size=(NB, Hkv, 2, bs)).astype(np.float32))
    ref_k, ref_v, ref_s = oracle.kv_write(rows[0], rows[1], slots, kc, vc, sc, layout="slot")
    gk, gv, gs = kc.cuda(), vc.cuda(), sc.cuda()
    say(f"[slot-major] writer bs={bs}")
    tq.tq_kv_write(rows[0].cuda(), rows[1].cuda(), torch.from_numpy(slots).cuda(), gk, gv, gs,
                   kv_layout="slot")
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy(), ref_k)
    assert np.array_equal(gv.cpu().numpy(), ref_v)
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    hk, hv, hs = (kc.permute(0, 2, 1, 3).contiguous().cuda(), vc.permute(0, 2, 1, 3).contiguous().cuda(),
                  sc.cuda())
    tq.tq_kv_write(rows[0].cuda(), rows[1].cuda(), torch.from_numpy(slots).cuda(), hk, hv, hs)
    torch.cuda.synchronize()
    assert torch.equal(hk.permute(0, 2, 1, 3).cpu(), gk.cpu())
    assert torch.equal(hv.permute(0, 2, 1, 3).cpu(), gv.cpu())


def test_slot_major_static_entry_point():
    """tq_decode_fused_static on a slot-major cache: the bits of the head-major call."""
    lens = (5000, 37, 3000, 8191)
    wl = workloads.small_workload(name="slotstatic", num_seqs=4, num_kv_heads=2, query_group_size=8,
                                  kv_block_size=32, seq_lens=lens, seed=97)
    head = workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=32)
    outs = []
    for inp in (head, head.with_layout("slot")):
        out = torch.empty((4, 16, 128), dtype=torch.bfloat16, device="cuda")
        tq.tq_decode_fused_static(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables,
                                  inp.seq_lens, out, 2, 8, 32, 1, inp.softmax_scale,
                                  num_partitions=32, max_seq_len=max(lens), kv_layout=inp.kv_layout)
        torch.cuda.synchronize()
        outs.append(out)
    say("[slot-major] static entry point")
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    compare(outs[1], oracle_decode(head), "static entry point, slot-major")
