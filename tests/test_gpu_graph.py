"""Both decode paths captured in a HIP graph (through torch's graph capture) and
replayed: between replays the inputs change in place (new queries, new sequence
lengths up to the captured max_seq_len) and eager work runs; every replay must
give the same bits as an eager call on the same inputs.  Needs an MI355X."""

import pytest
import torch

import paged_gqa_decode_amd as tq
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["two_kernel", "fused"])
def test_graph_replay_matches_eager(path):
    lens0 = (3000, 700, 4096, 1)
    wl = workloads.small_workload(name="graph", num_seqs=4, num_kv_heads=2, query_group_size=8,
                                  kv_block_size=32, seq_lens=lens0, seed=31)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=lens0, num_partitions=16)
    S, Hkv, QG, BS, G, P = 4, 2, 8, 32, 1, 16
    maxlen = 4096
    out = torch.empty((S, Hkv * QG, 128), dtype=torch.bfloat16, device="cuda")
    part = tq.alloc_partials(S, Hkv, P, QG, "cuda")
    # a workspace that makes the fused path split every (s, h) over several workgroups
    ws = torch.zeros(max(tq.fused_workspace_bytes(S, Hkv, QG, maxlen), 256), dtype=torch.uint8,
                     device="cuda")
    q = inp.q.clone()
    seq_lens = inp.seq_lens.clone()

    def step(stream=None):
        if path == "fused":
            tq.tq_decode_fused(q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables,
                               seq_lens, out, Hkv, QG, BS, G, inp.softmax_scale, num_partitions=P,
                               max_seq_len=maxlen, workspace=ws, stream=stream)
        else:
            tq.tq_decode(q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, seq_lens,
                         part, Hkv, QG, BS, G, inp.softmax_scale, num_partitions=P,
                         max_seq_len=maxlen, stream=stream)
            tq.tq_decode_reduce(part, seq_lens, out, Hkv, QG, G, num_partitions=P,
                                max_seq_len=maxlen, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"[graph] capture {path}")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep, lens in enumerate(((3000, 700, 4096, 1), (1, 4096, 17, 2500), (4096, 0, 333, 4000))):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        say(f"[graph] replay {rep} {path} lens={lens}")
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.fill_(float("nan"))  # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), out.view(torch.int16)), f"replay {rep} differs"
        assert torch.isfinite(got.float()).all()
    if path == "fused":
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "counters must stay re-armed"


@pytest.mark.parametrize("path", ["two_kernel", "fused"])
def test_capture_at_length_one_without_host_lengths(path):
    """decode() captured while every sequence has one token, with no host-side lengths: the
    binding takes the block table's capacity as the bound, sizes the grid for it and reads
    nothing back.  Replays with longer lengths (up to the capacity, zero included) equal eager
    calls on the same inputs."""
    S, Hkv, QG, BS = 3, 2, 16, 16
    cap_lens = (2048, 2048, 2048)
    wl = workloads.small_workload(name="graph1", num_seqs=S, num_kv_heads=Hkv, query_group_size=QG,
                                  kv_block_size=BS, seq_lens=cap_lens, seed=37)
    inp = workloads.make_inputs(wl, device="cuda", seq_lens=cap_lens)
    capacity = int(inp.block_tables.shape[1]) * BS  # the table has room for 2048 tokens or more
    assert capacity >= 2048
    q = inp.q.clone()
    seq_lens = torch.ones(S, dtype=torch.int32, device="cuda")
    fused = path == "fused"
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"[graph] capture {path} at length 1")
    with torch.cuda.graph(graph):
        out = tq.decode(q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, seq_lens,
                        softmax_scale=inp.softmax_scale, fused=fused)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(9)
    for rep, lens in enumerate(((1, 1, 1), (2048, 17, 0), (300, 2048, 1999), (256, 257, 2048))):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        say(f"[graph] replay {rep} {path} lens={lens}")
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = tq.decode(q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, seq_lens,
                        softmax_scale=inp.softmax_scale, fused=fused, max_seq_len=capacity)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep} differs"
        for s_, L in enumerate(lens):
            if L == 0:
                assert (got[s_].float() == 0).all()


@pytest.mark.parametrize("path", ["two_kernel", "fused"])
def test_tq4_graph_replay_matches_eager(path):
    """The 4-bit record format's paths captured and replayed with new queries and lengths
    (zero and the captured bound included): every replay equals an eager call bit for bit."""
    lens0 = (2500, 1, 4096, 900, 64)
    S, Hkv, QG, BS, G, P = 5, 2, 16, 16, 2, 8
    maxlen = 4096
    wl = workloads.small_workload(name="graph4", num_seqs=S, num_kv_heads=Hkv, query_group_size=QG,
                                  kv_block_size=BS, seq_lens=lens0, tile_groups_per_partition=G,
                                  seed=41)
    inp = workloads.make_inputs_tq4(wl, device="cuda", seq_lens=lens0, num_partitions=P)
    out = torch.empty((S, Hkv * QG, 128), dtype=torch.bfloat16, device="cuda")
    part = tq.alloc_partials(S, Hkv, P, QG, "cuda")
    ws = torch.zeros(max(tq.fused_workspace_bytes(S, Hkv, QG, maxlen), 256), dtype=torch.uint8,
                     device="cuda")
    q = inp.q.clone()
    seq_lens = inp.seq_lens.clone()

    def step():
        if path == "fused":
            tq.tq4_decode_fused(q, inp.cache, inp.centroids, inp.block_tables, seq_lens, out, Hkv,
                                QG, BS, G, inp.softmax_scale, num_partitions=P, max_seq_len=maxlen,
                                workspace=ws)
        else:
            tq.tq4_decode(q, inp.cache, inp.centroids, inp.block_tables, seq_lens, part, Hkv, QG,
                          BS, G, inp.softmax_scale, num_partitions=P, max_seq_len=maxlen)
            tq.tq_decode_reduce(part, seq_lens, out, Hkv, QG, G, num_partitions=P,
                                max_seq_len=maxlen)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"[graph] capture 4-bit {path}")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(6)
    for rep, lens in enumerate(((2500, 1, 4096, 900, 64), (0, 4096, 31, 32, 4000),
                                (4096, 4096, 4096, 4096, 4096))):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        say(f"[graph] replay {rep} 4-bit {path} lens={lens}")
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), out.view(torch.int16)), f"replay {rep} differs"
        assert torch.isfinite(got.float()).all()
        for s_, L in enumerate(lens):
            if L == 0:
                assert (got[s_].float() == 0).all()
    if path == "fused":
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "counters must stay re-armed"
