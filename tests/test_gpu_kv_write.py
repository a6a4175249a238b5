"""The KV-cache writer on the GPU against the oracle's writer: codes and scales
bit for bit (the quantizer's integer decisions are taken in fp32 on both
sides), untouched slots unchanged, and the written cache decoded correctly.
Needs an MI355X."""

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_amd as tq
from gpu_util import compare, say

pytestmark = pytest.mark.gpu


def make_rows(T, Hkv, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((2, T, Hkv, 128), generator=g)
    x[0, 1] *= 1e-7                        # tiny rows: codes in the fp8 subnormal range
    x[1, 2, 0] = 0.0                       # an all-zero row
    x[0, 3, :, 7] = 300.0                  # outliers
    x[1, 4] *= torch.rand((Hkv, 128), generator=g) ** 8  # many values near zero
    x[0, 5, 0, 0:8] = -0.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("bs", [16, 32])
def test_kv_write_matches_oracle(bs):
    T, Hkv, NB = 300, 4, 64
    rows = make_rows(T, Hkv, seed=bs)
    rng = np.random.default_rng(bs)
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    slots[::17] = -1                       # padding tokens
    slots[5] = NB * bs + 3                 # outside the pool: skipped
    kc = torch.from_numpy(rng.integers(0, 256, size=(NB, Hkv, bs, 128), dtype=np.uint8))
    vc = torch.from_numpy(rng.integers(0, 256, size=(NB, Hkv, bs, 128), dtype=np.uint8))
    sc = torch.from_numpy(rng.uniform(1, 2, size=(NB, Hkv, 2, bs)).astype(np.float32))
    ref_k, ref_v, ref_s = oracle.kv_write(rows[0], rows[1], np.where(slots >= NB * bs, -1, slots),
                                          kc, vc, sc)
    gk, gv, gs = kc.cuda(), vc.cuda(), sc.cuda()
    say(f"[kv_write] bs={bs} T={T}")
    tq.tq_kv_write(rows[0].cuda(), rows[1].cuda(), torch.from_numpy(slots).cuda(), gk, gv, gs)
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy(), ref_k), "K codes differ from the oracle"
    assert np.array_equal(gv.cpu().numpy(), ref_v), "V codes differ from the oracle"
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32)), "scales differ"


def test_written_cache_decodes():
    """Write a whole context with the GPU writer, then decode it with both paths: the result
    matches the oracle's decode of the same cache."""
    S, Hkv, QG, BS, L = 3, 2, 8, 32, 900
    NB = S * ((L + BS - 1) // BS)
    rng = np.random.default_rng(9)
    perm = rng.permutation(NB).astype(np.int32)
    bt = perm.reshape(S, -1)
    tok_slots = np.concatenate([bt[s][np.arange(L) // BS] * BS + np.arange(L) % BS for s in range(S)])
    g = torch.Generator().manual_seed(9)
    kv = torch.randn((2, S * L, Hkv, 128), generator=g).to(torch.bfloat16).cuda()
    k = torch.zeros((NB, Hkv, BS, 128), dtype=torch.uint8, device="cuda")
    v = torch.zeros_like(k)
    sc = torch.zeros((NB, Hkv, 2, BS), dtype=torch.float32, device="cuda")
    say("[kv_write] fill a cache, then decode it")
    tq.tq_kv_write(kv[0], kv[1], torch.from_numpy(tok_slots.astype(np.int32)).cuda(), k, v, sc)
    q = torch.randn((S, Hkv * QG, 128), generator=g).to(torch.bfloat16).cuda()
    bt_t = torch.from_numpy(bt.copy()).cuda()
    lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
    ref = oracle.decode(q.cpu(), k.cpu(), v.cpu(), sc.cpu(), bt_t.cpu(), lens.cpu(),
                        float(np.float32(1 / np.sqrt(128))))
    for fused in (False, True):
        out = tq.decode(q, k, v, sc, bt_t, lens, max_seq_len=L, fused=fused)
        torch.cuda.synchronize()
        compare(out, ref, f"decode of the written cache, fused={fused}")


def test_kv_write_magnitudes_bit_exact():
    """Rows scaled by powers of two from 2^-120 to 2^100 (so that the per-row scale falls on
    both sides of the writer's one-division range, [2^-90, FLT_MAX]), each row's values spread
    over many binades, some exact zeros and negative zeros: codes and scales bit for bit
    against the oracle."""
    T, Hkv, bs = 2048, 4, 32
    NB = T * Hkv // bs + 8
    g = torch.Generator().manual_seed(77)
    x = torch.randn((2, T, Hkv, 128), generator=g)
    x *= torch.exp2(torch.randint(-20, 1, (2, T, Hkv, 128), generator=g).float())
    x *= torch.exp2(torch.randint(-120, 101, (2, T, Hkv, 1), generator=g).float())
    x[:, ::7, :, ::5] = 0.0
    x[:, ::11, :, ::9] = -0.0
    rows = x.to(torch.bfloat16)
    rng = np.random.default_rng(78)
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    kc = torch.zeros((NB, Hkv, bs, 128), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    sc = torch.zeros((NB, Hkv, 2, bs), dtype=torch.float32)
    ref_k, ref_v, ref_s = oracle.kv_write(rows[0], rows[1], slots, kc, vc, sc)
    gk, gv, gs = kc.cuda(), vc.cuda(), sc.cuda()
    say(f"[kv_write] magnitudes T={T}")
    tq.tq_kv_write(rows[0].cuda(), rows[1].cuda(), torch.from_numpy(slots).cuda(), gk, gv, gs)
    torch.cuda.synchronize()
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32)), "scales differ"
    assert np.array_equal(gk.cpu().numpy(), ref_k), "K codes differ from the oracle"
    assert np.array_equal(gv.cpu().numpy(), ref_v), "V codes differ from the oracle"
