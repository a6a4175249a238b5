"""tq_decode_fused_static (the entry point that allocates nothing: the library's static
scratch instead of a caller's workspace) against tq_decode_fused, called through the C ABI,
on consecutive calls of different sizes -- a large batch, a smaller one, then a larger one
again, whose counters then lie where the smaller call left partials if the counter region
were not fixed.  Each output must equal tq_decode_fused's bit for bit (the same split with
a zero-filled workspace of tq_fused_workspace_bytes()) and match the oracle.  Needs an MI355X."""

import pytest
import torch

import paged_gqa_decode_amd as tq
import workloads
from gpu_util import compare, oracle_decode, say

pytestmark = pytest.mark.gpu

# (num_seqs, kv heads, QG, BS, lengths seed, max length): the even split over 2048 waves with
# cross-workgroup merges; a small batch; a long-context batch of many (s, h); a batch past the
# even split's 1024-sequence limit (per-(s, h) workgroups, no scratch partials needed).
CASES = [(48, 4, 8, 32, 1, 6000), (3, 2, 16, 16, 2, 1500), (200, 8, 6, 32, 3, 3000),
         (1030, 1, 8, 16, 4, 600)]


def _inputs(S, Hkv, QG, BS, seed, max_len):
    import numpy as np

    rng = np.random.default_rng(900 + seed)
    lens = rng.integers(0, max_len + 1, size=S)
    lens[0] = max_len
    lens = tuple(int(x) for x in lens)
    wl = workloads.small_workload(name=f"static{seed}", num_seqs=S, num_kv_heads=Hkv,
                                  query_group_size=QG, kv_block_size=BS, seq_lens=lens,
                                  seed=910 + seed)
    P = -(-max_len // 256)
    return workloads.make_inputs(wl, device="cuda", seq_lens=lens, num_partitions=P), max_len, P


def _run(inp, maxlen, P, static):
    wl = inp.wl
    S, Hkv, QG, BS = wl.num_seqs, wl.num_kv_heads, wl.query_group_size, wl.kv_block_size
    out = torch.full((S, Hkv * QG, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    args = (inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, inp.seq_lens, out,
            Hkv, QG, BS, 1, inp.softmax_scale)
    if static:
        tq.tq_decode_fused_static(*args, num_partitions=P, max_seq_len=maxlen)
    else:
        ws = tq.alloc_fused_workspace(S, Hkv, QG, maxlen, "cuda")
        tq.tq_decode_fused(*args, num_partitions=P, max_seq_len=maxlen, workspace=ws)
    torch.cuda.synchronize()
    return out


def test_static_scratch_matches_workspace_path():
    for i, case in enumerate(CASES):
        inp, maxlen, P = _inputs(*case)
        say(f"[static scratch] call {i + 1}: S={case[0]} Hkv={case[1]} QG={case[2]} BS={case[3]} "
            f"max_len={maxlen}")
        got = _run(inp, maxlen, P, static=True)
        ref = _run(inp, maxlen, P, static=False)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), case
        compare(got, oracle_decode(inp), f"static scratch call {i + 1}")
        # a repeat of the same call on the scratch the previous call left: the same bits
        again = _run(inp, maxlen, P, static=True)
        assert torch.equal(again.view(torch.int16), got.view(torch.int16)), case
