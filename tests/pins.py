"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises (AssertionError or
OracleError) when that build of the oracle disagrees with:
  * the e4m3fn / bf16 format definitions (closed-form code values) and torch's
    own fp8 / bf16 conversions (a library routine, run, not retyped);
  * brute-force dense attention computed with torch float64 library ops
    (softmax, matmul, scaled_dot_product_attention) over a gather written
    here, on tiny inputs;
  * closed forms: one cached token returns its V row; a zero query returns
    the mean of V; constant V returns V; a hand-derived two-token example;
  * invariants: physical-block permutation with a consistent table, split-K
    merge == unsplit for many partition counts, V-scale linearity, an
    isolated dominant token returns that token's V row, tables that share
    blocks equal a copy with the shared blocks duplicated, scales of either
    sign.

``test_oracle_pins.py`` runs them against the oracle; ``test_oracle_mutants.py``
plants plausible mistakes in copies of oracle.c and checks that every planted
mistake fails at least one pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# tiny problem builder (test-local, independent of the generator module)
# ----------------------------------------------------------------------------

def tiny_problem(S=3, Hkv=2, QG=4, D=32, BS=4, lens=(1, 7, 13), extra_blocks=3, seed=0,
                 max_blocks=None):
    rng = np.random.default_rng(seed)
    need = [-(-L // BS) for L in lens]
    NB = sum(need) + extra_blocks
    MB = max_blocks or max(max(need), 1) + 1
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.zeros((S, MB), dtype=np.int32)
    pos = 0
    for s in range(S):
        bt[s, :need[s]] = perm[pos:pos + need[s]]
        pos += need[s]
    q = torch.from_numpy(rng.standard_normal((S, Hkv * QG, D)).astype(np.float32)).to(torch.bfloat16)
    def codes():
        x = torch.from_numpy(rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32) * 100)
        return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    k = codes()
    v = codes()
    sc = torch.from_numpy(rng.uniform(0.001, 0.02, size=(NB, Hkv, 2, BS)).astype(np.float32))
    sl = torch.tensor(lens, dtype=torch.int32)
    return dict(q=q, k=k, v=v, sc=sc, bt=torch.from_numpy(bt), sl=sl,
                scale=float(np.float32(1.0 / math.sqrt(D))))


def dense_rows(p, s, h, field):
    """Gathered, dequantized K (field 0) or V (field 1) rows of (s, h) as float64 [L][D]."""
    cache = p["k"] if field == 0 else p["v"]
    BS = cache.shape[2]
    L = int(p["sl"][s])
    rows = []
    for t in range(L):
        b = int(p["bt"][s, t // BS])
        j = t % BS
        vals = cache[b, h, j].view(torch.float8_e4m3fn).to(torch.float64)
        rows.append(vals * float(p["sc"][b, h, field, j]))
    D = cache.shape[3]
    return torch.stack(rows) if rows else torch.zeros((0, D), dtype=torch.float64)


def run(orc, p, **kw):
    return orc.decode(p["q"], p["k"], p["v"], p["sc"], p["bt"], p["sl"], p["scale"], **kw)


def assert_close(a, b, rel, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= rel * ref, f"{what}: max abs err {err:.3e} > {rel:.1e} * {ref:.3e}"


# ----------------------------------------------------------------------------
# format pins
# ----------------------------------------------------------------------------

def pin_e4m3fn_points(orc):
    """Closed-form values of the OCP e4m3fn format: bias 7, 3 mantissa bits, no inf."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
            0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0,
            0x81: -(2.0 ** -9)}
    got = orc.dec_e4m3fn(np.array(sorted(want), dtype=np.uint8))
    for c, g in zip(sorted(want), got):
        assert g == want[c], f"code {c:#x}: {g} != {want[c]}"
    nan = orc.dec_e4m3fn(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan)), "0x7F / 0xFF must decode to NaN"
    neg0 = orc.dec_e4m3fn(np.array([0x80], dtype=np.uint8))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0, "0x80 is -0"
    pos = orc.dec_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    negs = orc.dec_e4m3fn(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(negs, -pos), "sign bit must negate"


def pin_e4m3fn_library(orc):
    """All 256 codes against torch's float8_e4m3fn -> float64 conversion."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.dec_e4m3fn(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"e4m3fn mismatch at codes {np.nonzero(~same)[0][:8]}"


def pin_bf16_library(orc):
    """bfloat16 bit patterns against torch's bfloat16 -> float64 conversion."""
    rng = np.random.default_rng(7)
    bits = np.concatenate([rng.integers(0, 1 << 16, size=4000), [0, 0x8000, 0x3F80, 0xBF80, 0x7F7F,
                                                                 0x0001, 0x0080, 0x7F80, 0xFF80]])
    bits = bits.astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.dec_bf16(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "bf16 decode mismatch"


# ----------------------------------------------------------------------------
# attention pins
# ----------------------------------------------------------------------------

def _bruteforce(p):
    S, Hq, D = p["q"].shape
    Hkv = p["k"].shape[1]
    QG = Hq // Hkv
    out = torch.zeros((S, Hq, D), dtype=torch.float64)
    for s in range(S):
        if int(p["sl"][s]) == 0:
            continue
        for h in range(Hkv):
            K = dense_rows(p, s, h, 0)
            V = dense_rows(p, s, h, 1)
            Q = p["q"][s, h * QG:(h + 1) * QG].to(torch.float64)
            logits = (Q @ K.T) * p["scale"]
            out[s, h * QG:(h + 1) * QG] = torch.softmax(logits, dim=-1) @ V
    return out.numpy()


def pin_dense_bruteforce(orc):
    """Against softmax(q K^T * scale) V with torch float64 ops on gathered rows."""
    for seed, kw in ((0, {}), (1, dict(BS=8, lens=(9, 16, 1), QG=6)), (2, dict(S=2, Hkv=3, QG=2, lens=(40, 3)))):
        p = tiny_problem(seed=seed, **kw)
        assert_close(run(orc, p), _bruteforce(p), 1e-12, f"bruteforce seed {seed}")


def pin_sdpa(orc):
    """Against torch.nn.functional.scaled_dot_product_attention in float64."""
    p = tiny_problem(S=2, Hkv=2, QG=3, D=64, BS=16, lens=(33, 50), seed=5)
    got = run(orc, p)
    for s in range(2):
        for h in range(2):
            K = dense_rows(p, s, h, 0)[None]
            V = dense_rows(p, s, h, 1)[None]
            Q = p["q"][s, h * 3:(h + 1) * 3].to(torch.float64)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=p["scale"])[0]
            assert_close(got[s, h * 3:(h + 1) * 3], ref.numpy(), 1e-12, "sdpa")


def pin_single_token(orc):
    """One cached token: the output is exactly that token's dequantized V row."""
    p = tiny_problem(S=2, Hkv=2, QG=3, lens=(1, 1), seed=3)
    got = run(orc, p)
    for s in range(2):
        for h in range(2):
            v0 = dense_rows(p, s, h, 1)[0].numpy()
            for g in range(3):
                assert np.array_equal(got[s, h * 3 + g], v0), "L=1 must return v_0 exactly"


def pin_zero_query(orc):
    """q = 0: all logits 0, the output is the mean of the V rows."""
    p = tiny_problem(seed=4, lens=(5, 12, 30))
    p["q"] = torch.zeros_like(p["q"])
    got = run(orc, p)
    QG = 4
    for s in range(3):
        for h in range(2):
            mean = dense_rows(p, s, h, 1).mean(dim=0).numpy()
            for g in range(QG):
                assert_close(got[s, h * QG + g], mean, 1e-13, "q=0 mean")


def pin_constant_v(orc):
    """V rows all equal: the output is that row whatever the weights."""
    p = tiny_problem(seed=6, lens=(3, 17, 25))
    p["v"] = torch.full_like(p["v"], 0x44)  # 3.0
    p["sc"][:, :, 1, :] = 0.25
    got = run(orc, p)
    assert_close(got, np.full(got.shape, 0.75), 1e-14, "constant V")


def pin_two_token_golden(orc):
    """The hand-derived worked example stored under tests/golden/."""
    with open(os.path.join(GOLDEN, "two_token_example.json")) as f:
        ex = json.load(f)
    D, BS = ex["head_dim"], ex["kv_block_size"]
    q = torch.zeros((1, 1, D), dtype=torch.int16)
    q[0, 0, 0] = ex["q_d0_bf16_bits"]
    q = q.view(torch.bfloat16)
    k = torch.zeros((1, 1, BS, D), dtype=torch.uint8)
    k[0, 0, 1, 0] = ex["k_token1_d0_code"]
    v = torch.zeros((1, 1, BS, D), dtype=torch.uint8)
    v[0, 0, 0, :] = ex["v_token0_code"]
    v[0, 0, 1, :] = ex["v_token1_code"]
    sc = torch.ones((1, 1, 2, BS), dtype=torch.float32)
    sc[0, 0, 1, 0] = ex["v_token0_scale"]
    sc[0, 0, 1, 1] = ex["v_token1_scale"]
    out = orc.decode(q, k, v, sc, torch.zeros((1, 1), dtype=torch.int32),
                     torch.tensor([2], dtype=torch.int32), 1.0)
    want = (2 - math.e / 2) / (1 + math.e)
    assert abs(want - ex["expected_value"]) < 1e-15
    assert_close(out[0, 0], np.full(D, want), 1e-14, "two-token closed form")


def pin_block_permutation(orc):
    """Relabel physical blocks (move the data, rewrite the table): bit-identical output."""
    p = tiny_problem(seed=8, lens=(13, 29, 4), BS=4)
    ref = run(orc, p)
    NB = p["k"].shape[0]
    perm = torch.from_numpy(np.random.default_rng(9).permutation(NB).astype(np.int64))
    q = dict(p)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(NB)
    q["k"] = p["k"][inv].contiguous()  # new block perm[b] holds old block b
    q["v"] = p["v"][inv].contiguous()
    q["sc"] = p["sc"][inv].contiguous()
    q["bt"] = perm[p["bt"].long()].to(torch.int32)
    got = run(orc, q)
    assert np.array_equal(got, ref), "block permutation changed the output bits"


def pin_split_merge(orc):
    """Split-K partials merged by log-sum-exp equal the unsplit result for any partition count."""
    p = tiny_problem(seed=10, lens=(1, 37, 64, 95), S=4, BS=4, max_blocks=25)
    ref = run(orc, p)
    for P, E in ((1, 100), (2, 48), (3, 32), (7, 14), (32, 3), (95, 1), (13, 8)):
        o, m, l = orc.partials(p["q"], p["k"], p["v"], p["sc"], p["bt"], p["sl"], p["scale"], P, E)
        sl = p["sl"].numpy()
        for s, L in enumerate(sl):
            live = -(-int(L) // E)
            assert np.all(np.isfinite(m[s, :, :live])) and np.all(np.isnan(m[s, :, live:])), "live/dead"
            assert np.all(l[s, :, :live] >= 1.0), "l_p >= 1 (the max term contributes exp(0))"
        out = orc.merge(o, m, l, p["sl"], E)
        assert_close(out, ref, 1e-13, f"split merge P={P} E={E}")


def pin_partials_closed_form(orc):
    """Each partial of the split-K triple against its definition, computed independently per
    partition with torch float64 on gathered rows: m_p = max over the partition's tokens of the
    scaled logit x = scale * q.k (natural-log units, as the page's STEP G defines them), l_p =
    sum exp(x - m_p), o_p = sum exp(x - m_p) v / l_p; dead partitions stay NaN.  With one token
    per partition this is m_p = x_t, l_p = 1, o_p = v_t."""
    p = tiny_problem(seed=12, lens=(1, 9, 14), S=3, BS=4, max_blocks=6)
    S, Hq, D = p["q"].shape
    Hkv = p["k"].shape[1]
    QG = Hq // Hkv
    for P, E in ((14, 1), (5, 3), (2, 7)):
        o, m, l = orc.partials(p["q"], p["k"], p["v"], p["sc"], p["bt"], p["sl"], p["scale"], P, E)
        for s in range(S):
            L = int(p["sl"][s])
            for h in range(Hkv):
                K = dense_rows(p, s, h, 0)
                V = dense_rows(p, s, h, 1)
                Q = p["q"][s, h * QG:(h + 1) * QG].to(torch.float64)
                x = (Q @ K.T) * p["scale"]  # [QG][L]
                for pp in range(P):
                    t0, t1 = pp * E, min((pp + 1) * E, L)
                    if t0 >= L:
                        assert np.all(np.isnan(m[s, h, pp])), "dead partition written"
                        continue
                    xp = x[:, t0:t1]
                    mp = xp.max(dim=1).values
                    w = torch.exp(xp - mp[:, None])
                    lp = w.sum(dim=1)
                    op = (w @ V[t0:t1]) / lp[:, None]
                    assert_close(m[s, h, pp], mp.numpy(), 1e-13, f"m_p P={P} E={E}")
                    assert_close(l[s, h, pp], lp.numpy(), 1e-13, f"l_p P={P} E={E}")
                    assert_close(o[s, h, pp], op.numpy(), 1e-13, f"o_p P={P} E={E}")
                    if t1 - t0 == 1:
                        assert np.all(l[s, h, pp] == 1.0), "one token: l_p = exp(0) = 1 exactly"


def pin_v_scale_linearity(orc):
    """Doubling every V scale doubles the output exactly (power-of-two scaling)."""
    p = tiny_problem(seed=11, lens=(6, 19, 2))
    ref = run(orc, p)
    p2 = dict(p)
    sc = p["sc"].clone()
    sc[:, :, 1, :] *= 2
    p2["sc"] = sc
    assert np.array_equal(run(orc, p2), 2 * ref)


def pin_dominant_token(orc):
    """K zero except at token t* where K is parallel to q (logit margin >= 80): out = V[t*]."""
    D, BS, Hkv, QG = 32, 4, 2, 2
    L = 23
    for tstar in (0, 3, 4, 11, 22):
        p = tiny_problem(S=1, Hkv=Hkv, QG=QG, D=D, BS=BS, lens=(L,), seed=12)
        q = torch.zeros((1, Hkv * QG, D))
        q[0, :, :] = 1.0
        p["q"] = q.to(torch.bfloat16)
        k = torch.zeros_like(p["k"])
        b = int(p["bt"][0, tstar // BS])
        k[b, :, tstar % BS, :] = 0x48  # 4.0
        p["k"] = k
        p["sc"][:, :, 0, :] = 1.0
        p["scale"] = 1.0  # logit of t* = 128, others 0
        got = run(orc, p)
        for h in range(Hkv):
            vt = dense_rows(p, 0, h, 1)[tstar].numpy()
            for g in range(QG):
                assert_close(got[0, h * QG + g], vt, 1e-30, f"dominant token t*={tstar}")


def pin_aliased_blocks(orc):
    """Tables that share physical blocks (prefix sharing: one sequence's first blocks named by
    another's table, one block named by every entry of a table): the oracle against the
    brute-force gather + softmax, and bit for bit against a copy in which every shared block
    is duplicated so that no two entries name the same block."""
    p = tiny_problem(S=4, lens=(13, 13, 6, 20), BS=4, seed=14, extra_blocks=2, max_blocks=6)
    bt = p["bt"].clone()
    bt[1, :3] = bt[0, :3]      # sequence 1 shares its first 3 blocks with sequence 0
    bt[2, :2] = bt[0, :2]      # sequence 2 lies inside sequence 0's blocks
    bt[3, :5] = bt[3, 0]       # every entry of sequence 3 names one block
    p["bt"] = bt
    got = run(orc, p)
    assert_close(got, _bruteforce(p), 1e-12, "aliased bruteforce")
    NB = p["k"].shape[0]
    seen, extra = set(), []
    bt2 = bt.clone()
    for s, L in enumerate(p["sl"].tolist()):
        for j in range(-(-L // 4)):
            b = int(bt[s, j])
            if b in seen:
                bt2[s, j] = NB + len(extra)
                extra.append(b)
            seen.add(b)
    assert extra
    src = torch.tensor(extra, dtype=torch.int64)
    q = dict(p, bt=bt2, k=torch.cat([p["k"], p["k"][src]]), v=torch.cat([p["v"], p["v"][src]]),
             sc=torch.cat([p["sc"], p["sc"][src]]))
    assert np.array_equal(run(orc, q), got), "duplicating shared blocks changed the output"


def pin_signed_scales(orc):
    """K and V scales of either sign (code * scale, whatever the sign): against the brute-force
    gather + softmax; negating every V scale negates the output exactly."""
    p = tiny_problem(seed=15, lens=(9, 26, 3))
    rng = np.random.default_rng(16)
    p["sc"] = p["sc"] * torch.from_numpy(rng.choice([-1.0, 1.0], size=p["sc"].shape).astype(np.float32))
    got = run(orc, p)
    assert_close(got, _bruteforce(p), 1e-12, "signed scales bruteforce")
    sc = p["sc"].clone()
    sc[:, :, 1, :] = -sc[:, :, 1, :]
    assert np.array_equal(run(orc, dict(p, sc=sc)), -got)


def _slot_major(x):
    """A head-major [NB][Hkv][BS][...] cache array as the slot-major [NB][BS][Hkv][...] one."""
    return x.permute(0, 2, 1, 3).contiguous()


def pin_slot_major_transposition(orc):
    """The same cache in the slot-major row order (the page's data region) decodes, splits and
    merges to the same bits as in the head-major order (pinned by the brute-force gather), and
    the slot-major rows match a gather written here from the page's byte formula."""
    for seed, kw in ((30, dict(lens=(5, 13, 22), BS=4)), (31, dict(S=2, Hkv=3, QG=2, BS=8, lens=(17, 40)))):
        p = tiny_problem(seed=seed, **kw)
        k2, v2 = _slot_major(p["k"]), _slot_major(p["v"])
        ref = run(orc, p)
        got = orc.decode(p["q"], k2, v2, p["sc"], p["bt"], p["sl"], p["scale"], layout="slot")
        assert np.array_equal(got, ref), "slot-major decode differs from head-major"
        o, m, l = orc.partials(p["q"], p["k"], p["v"], p["sc"], p["bt"], p["sl"], p["scale"], 6, 8)
        o2, m2, l2 = orc.partials(p["q"], k2, v2, p["sc"], p["bt"], p["sl"], p["scale"], 6, 8,
                                  layout="slot")
        for a, b in ((o, o2), (m, m2), (l, l2)):
            assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0))
        # gather from the flat slot-major bytes: byte (b, j, h, d) = b*BS*Hkv*D + j*Hkv*D + h*D + d
        NB, Hkv, BS, D = p["k"].shape
        flat_k, flat_v = k2.reshape(-1), v2.reshape(-1)
        S, Hq, _ = p["q"].shape
        QG = Hq // Hkv
        want = np.zeros((S, Hq, D))
        for s in range(S):
            L = int(p["sl"][s])
            for h in range(Hkv):
                rows = []
                for t in range(L):
                    b, j = int(p["bt"][s, t // BS]), t % BS
                    at = b * BS * Hkv * D + j * Hkv * D + h * D
                    kv = [c[at:at + D].view(torch.float8_e4m3fn).to(torch.float64)
                          * float(p["sc"][b, h, f, j]) for f, c in ((0, flat_k), (1, flat_v))]
                    rows.append(kv)
                if not rows:
                    continue
                K = torch.stack([r[0] for r in rows])
                V = torch.stack([r[1] for r in rows])
                Q = p["q"][s, h * QG:(h + 1) * QG].to(torch.float64)
                want[s, h * QG:(h + 1) * QG] = (torch.softmax(Q @ K.T * p["scale"], -1) @ V).numpy()
        assert_close(got, want, 1e-12, "slot-major gather")


def pin_two_token_slot_major_golden(orc):
    """tests/golden/two_token_slot_major.json: the two-token closed form, its bytes placed by
    hand at the offsets of the page's slot-major data region."""
    with open(os.path.join(GOLDEN, "two_token_slot_major.json")) as f:
        g = json.load(f)
    z = g["sizes"]
    NB, BS, Hkv, D = z["num_blocks"], z["kv_block_size"], z["num_kv_heads"], z["head_dim"]
    k = np.zeros(NB * BS * Hkv * D, dtype=np.uint8)
    v = np.zeros_like(k)
    for off, val in g["k_bytes"].items():
        k[int(off)] = val
    for off, val in g["v_bytes"].items():
        v[int(off)] = val
    sc = np.ones(NB * Hkv * 2 * BS, dtype=np.float32)
    for off, val in g["scale_overrides"].items():
        sc[int(off)] = val
    q = np.zeros((1, Hkv, D), dtype=np.uint16)
    q[0, 1, 0] = g["q_head1_d0_bf16_bits"]
    out = orc.decode(q, k.reshape(NB, BS, Hkv, D), v.reshape(NB, BS, Hkv, D),
                     sc.reshape(NB, Hkv, 2, BS), np.array([[1]], dtype=np.int32),
                     np.array([2], dtype=np.int32), 1.0, layout="slot")
    want = (2 - math.e / 2) / (1 + math.e)
    assert abs(want - g["expected_head1_value"]) < 1e-15
    assert_close(out[0, 1], np.full(D, want), 1e-14, "slot-major two-token closed form")
    assert not out[0, 0].any()


def pin_tq4_golden_record_slot_major(orc):
    """tests/golden/tq4_record_slot_major.json: a record written byte by byte at offsets
    derived by hand from the page's slot-major data region, dequantized, then a 3-token
    decode over it (q = 0: the mean of the V rows; q = e_0: a closed-form softmax)."""
    with open(os.path.join(GOLDEN, "tq4_record_slot_major.json")) as f:
        g = json.load(f)
    sz = g["sizes"]
    NB, Hkv, BS, D = sz["num_blocks"], sz["num_kv_heads"], sz["kv_block_size"], sz["head_dim"]
    cache = np.zeros(NB * sz["block_bytes"], dtype=np.uint8)
    for off, val in g["bytes"].items():
        cache[int(off)] = val
    cache = cache.reshape(NB, sz["block_bytes"])
    cent = np.asarray(g["centroids"], dtype=np.float32)
    rec = g["record"]
    k, v = orc.dequant_tq4(cache, cent, Hkv, D, BS, rec["block"], rec["head"], rec["slot"],
                           layout="slot")
    assert np.array_equal(k, np.asarray(g["expected_k"])), k
    assert np.array_equal(v, np.asarray(g["expected_v"])), v
    for (b, h, slot) in ((1, 0, 2), (1, 1, 1), (0, 1, 2)):
        k0, v0 = orc.dequant_tq4(cache, cent, Hkv, D, BS, b, h, slot, layout="slot")
        assert not k0.any() and not v0.any()
    bt = np.array([[1]], dtype=np.int32)
    sl = np.array([3], dtype=np.int32)
    q = np.zeros((1, Hkv, D), dtype=np.uint16)
    out = orc.decode_tq4(q, cache, cent, bt, sl, 1.0, Hkv, BS, layout="slot")
    assert np.array_equal(out[0, 1], np.asarray(g["expected_v"]) / 3)
    assert not out[0, 0].any()
    q[0, 1, 0] = 0x3F80
    out = orc.decode_tq4(q, cache, cent, bt, sl, 1.0, Hkv, BS, layout="slot")
    w = math.exp(-14.0)
    assert np.max(np.abs(out[0, 1] - np.asarray(g["expected_v"]) * w / (w + 2.0))) < 1e-15


def pin_tq4_slot_major_transposition(orc):
    """A 4-bit cache whose data rows are reordered head-major -> slot-major (metadata
    untouched) decodes to the same bits with layout "slot"."""
    p = _tq4_problem(6)
    NB, Hkv, BS, D = p["cache"].shape[0], p["Hkv"], p["BS"], 128
    data = p["cache"][:, :Hkv * BS * D].reshape(NB, Hkv, BS, D).transpose(0, 2, 1, 3).reshape(NB, -1)
    cache2 = np.ascontiguousarray(np.concatenate([data, p["cache"][:, Hkv * BS * D:]], axis=1))
    a = orc.decode_tq4(p["q"], p["cache"], p["cent"], p["bt"], p["sl"], 0.088, Hkv, BS)
    b = orc.decode_tq4(p["q"], cache2, p["cent"], p["bt"], p["sl"], 0.088, Hkv, BS, layout="slot")
    assert np.array_equal(a, b)


def pin_kv_write_slot_major(orc):
    """The writer into a slot-major cache leaves exactly the transposition of what it leaves in
    the head-major one (codes; the scale region is the same in both)."""
    kn, vn, sm, kc, vc, sc = _kv_write_problem(seed=5)
    a = orc.kv_write(kn, vn, sm, kc, vc, sc)
    b = orc.kv_write(kn, vn, sm, _slot_major(torch.from_numpy(kc)).numpy(),
                     _slot_major(torch.from_numpy(vc)).numpy(), sc, layout="slot")
    assert np.array_equal(_slot_major(torch.from_numpy(a[0])).numpy(), b[0])
    assert np.array_equal(_slot_major(torch.from_numpy(a[1])).numpy(), b[1])
    assert np.array_equal(a[2], b[2])


def pin_zero_length(orc):
    p = tiny_problem(seed=13, lens=(0, 5, 0))
    got = run(orc, p)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.any(got[1] != 0)


# ----------------------------------------------------------------------------
# KV-cache writer pins (quantize + scatter)
# ----------------------------------------------------------------------------

def pin_e4m3fn_encode_roundtrip(orc):
    """Every finite code encodes back to itself from its own value."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = orc.dec_e4m3fn(codes).astype(np.float32)
    assert np.array_equal(orc.enc_e4m3fn(vals), codes)


def pin_e4m3fn_encode_ties_and_saturation(orc):
    """Midpoints between neighbouring codes go to the even code; just off a midpoint goes to the
    nearer code; magnitudes above 448 saturate to 448 (0x7E / 0xFE)."""
    pos = orc.dec_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8))
    for c in range(0, 0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)  # exact in fp32
        want_even = c if c % 2 == 0 else c + 1
        assert orc.enc_e4m3fn([mid])[0] == want_even, f"tie between {c:#x} and {c + 1:#x}"
        lo = np.nextafter(mid, np.float32(0))
        hi = np.nextafter(mid, np.float32(1000))
        assert orc.enc_e4m3fn([lo])[0] == c and orc.enc_e4m3fn([hi])[0] == c + 1
    sat = orc.enc_e4m3fn(np.array([448.0, 449.0, 464.0, 480.0, 1e30, -500.0, -1e30], np.float32))
    assert list(sat) == [0x7E] * 5 + [0xFE] * 2
    assert orc.enc_e4m3fn([np.float32(-0.0)])[0] == 0x80


def pin_e4m3fn_encode_library(orc):
    """Random fp32 values within +-448 (subnormal fp8 range included) against torch's
    round-to-nearest-even float8_e4m3fn cast."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.02, 0.02, 2000),
                        rng.standard_normal(2000) * 10]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.enc_e4m3fn(v), ref)


def _kv_write_problem(seed=0, T=5, Hkv=3, D=128, BS=16, NB=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, T, Hkv, D)).astype(np.float32)
    x[0, 1, 0] *= 1e-6      # a tiny row: codes land in the fp8 subnormal range after scaling
    x[1, 2, 1] = 0.0        # an all-zero row: scale 0, codes 0
    x[0, 3, 2, 5] = 300.0   # an outlier
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = rng.permutation(NB * BS)[:T].astype(np.int32)
    slots[4] = -1           # padding token: skipped
    kc = rng.integers(0, 256, size=(NB, Hkv, BS, D), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(NB, Hkv, BS, D), dtype=np.uint8)
    sc = rng.uniform(1, 2, size=(NB, Hkv, 2, BS)).astype(np.float32)
    return bits[0], bits[1], slots, kc, vc, sc


def pin_kv_write_quantizer(orc):
    """Written rows: scale = fp32(absmax / 448); the max element maps to +-448; every value is
    within half a code step (RNE); zero rows give scale 0, codes 0; skipped tokens and other
    slots are untouched."""
    kn, vn, slots, kc, vc, sc = _kv_write_problem()
    kc2, vc2, sc2 = orc.kv_write(kn, vn, slots, kc, vc, sc)
    NB, Hkv, BS, D = kc.shape
    written = np.zeros((NB, Hkv, BS), dtype=bool)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), BS)
        for h in range(Hkv):
            written[blk, h, off] = True
            for field, (bits, cache) in enumerate(((kn, kc2), (vn, vc2))):
                x = torch.from_numpy(bits[t, h].view(np.int16)).view(torch.bfloat16).float().numpy()
                s = sc2[blk, h, field, off]
                assert s == np.float32(np.abs(x).max()) / np.float32(448.0)
                codes = cache[blk, h, off]
                if s == 0:
                    assert not codes.any()
                    continue
                deq = orc.dec_e4m3fn(codes) * np.float64(s)
                q = np.abs(x.astype(np.float64) / s)
                step = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 1e-300))) - 3),
                                2.0 ** -9)
                assert np.all(np.abs(deq - x) <= 0.5 * step * s * (1 + 1e-6) + 1e-30)
                assert np.abs(orc.dec_e4m3fn(codes)).max() == 448.0
    keep = ~written
    assert np.array_equal(kc2[keep], kc[keep]) and np.array_equal(vc2[keep], vc[keep])
    assert np.array_equal(sc2[:, :, 0][keep], sc[:, :, 0][keep])
    assert np.array_equal(sc2[:, :, 1][keep], sc[:, :, 1][keep])


def pin_kv_write_matches_library_quantizer(orc):
    """The same rows quantized with torch ops (fp32 division, clamp, torch's RNE fp8 cast) give
    the same codes and scales."""
    kn, vn, slots, kc, vc, sc = _kv_write_problem(seed=4)
    kc2, vc2, sc2 = orc.kv_write(kn, vn, slots, kc, vc, sc)
    BS = kc.shape[2]
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), BS)
        for field, (bits, cache) in enumerate(((kn, kc2), (vn, vc2))):
            x = torch.from_numpy(bits[t].view(np.int16)).view(torch.bfloat16).float()  # [Hkv][D]
            s = x.abs().amax(dim=-1) / 448.0
            div = torch.where(s > 0, s, torch.ones_like(s))
            codes = (x / div[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
            codes = torch.where(s[:, None] > 0, codes, torch.zeros_like(codes))
            assert np.array_equal(cache[blk, :, off], codes.numpy())
            assert np.array_equal(sc2[blk, :, field, off], s.numpy())


# ----------------------------------------------------------------------------
# The 4-bit record format
# ----------------------------------------------------------------------------

def pin_f16_library(orc):
    """All 65536 fp16 bit patterns against numpy's float16 (NaN patterns decode to NaN)."""
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.dec_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    live = ~np.isnan(ref)
    assert np.array_equal(got[live], ref[live])


def pin_tq4_golden_record(orc):
    """The hand-written record of tests/golden/tq4_record.json: its bytes sit at offsets
    derived by hand from the layout, and its dequantized K and V rows are derived by hand.
    Then a 4-token sequence whose other records are zero: with q = 0 the output is the mean
    of the V rows; with q = e_0 a 4-token softmax in closed form."""
    with open(os.path.join(GOLDEN, "tq4_record.json")) as f:
        g = json.load(f)
    sz = g["sizes"]
    NB, Hkv, BS, D = sz["num_blocks"], sz["num_kv_heads"], sz["kv_block_size"], sz["head_dim"]
    cache = np.zeros(NB * sz["block_bytes"], dtype=np.uint8)
    for off, val in g["bytes"].items():
        cache[int(off)] = val
    cache = cache.reshape(NB, sz["block_bytes"])
    cent = np.asarray(g["centroids"], dtype=np.float32)
    rec = g["record"]
    k, v = orc.dequant_tq4(cache, cent, Hkv, D, BS, rec["block"], rec["head"], rec["slot"])
    assert np.array_equal(k, np.asarray(g["expected_k"])), k
    assert np.array_equal(v, np.asarray(g["expected_v"])), v
    # every other record of the cache is zero bytes: index 0 with zero norm, scale and zero point
    for (b, h, slot) in ((0, 0, 0), (1, 1, 2), (1, 0, 3)):
        k0, v0 = orc.dequant_tq4(cache, cent, Hkv, D, BS, b, h, slot)
        assert not k0.any() and not v0.any()
    # sequence of 4 tokens in block 1: slots 0..3, the record is token 3 of kv head 1
    bt = np.array([[1]], dtype=np.int32)
    sl = np.array([4], dtype=np.int32)
    q = np.zeros((1, Hkv, D), dtype=np.uint16)  # QG = 1
    out = orc.decode_tq4(q, cache, cent, bt, sl, 1.0, Hkv, BS)
    assert np.array_equal(out[0, 1], np.asarray(g["expected_v"]) / 4)
    assert not out[0, 0].any()
    q[0, 1, 0] = 0x3F80  # bf16 1.0 at dim 0: x_3 = k[0] = -14, the other logits 0
    out = orc.decode_tq4(q, cache, cent, bt, sl, 1.0, Hkv, BS)
    w = math.exp(-14.0)
    want = np.asarray(g["expected_v"]) * w / (w + 3.0)
    assert np.max(np.abs(out[0, 1] - want)) < 1e-15


_E4M3_EXACT_CENTROIDS = [-6.0, -4.0, -3.0, -2.0, -1.5, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 1.5, 2.0,
                         3.0, 4.0, 6.0]


def _tq4_problem(seed, v_const=None, v_scale=None, v_zero=None):
    """A small random problem in the 4-bit format, with the arrays of an equivalent fp8
    cache when every dequantized value is e4m3-exact (centroids e4m3-exact, norms and V
    scales powers of two, zero point 0)."""
    import workloads

    rng = np.random.default_rng(seed)
    S, Hkv, QG, D, BS = 3, 2, 4, 128, 16
    lens = np.array([5, 16, 40], dtype=np.int32)
    need = [-(-int(L) // BS) for L in lens]
    NB = sum(need) + 2
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.zeros((S, max(need) + 1), dtype=np.int32)
    pos = 0
    for s_, n in enumerate(need):
        bt[s_, :n] = perm[pos:pos + n]
        pos += n
    k_idx = rng.integers(0, 16, size=(NB, Hkv, BS, D), dtype=np.uint8)
    v_idx = rng.integers(0, 16, size=(NB, Hkv, BS, D), dtype=np.uint8)
    if v_const is not None:
        v_idx[:] = v_const
    knorm = np.ldexp(1.0, rng.integers(-3, 4, size=(NB, Hkv, BS))).astype(np.float16)
    if v_scale is None:
        vscale = np.ldexp(1.0, rng.integers(-3, 4, size=(NB, Hkv, BS))).astype(np.float16)
    else:
        vscale = np.full((NB, Hkv, BS), v_scale, dtype=np.float16)
    vzero = np.full((NB, Hkv, BS), 0.0 if v_zero is None else v_zero, dtype=np.float16)
    meta = np.stack([knorm, vscale, vzero], axis=2).view(np.int16)  # [NB][Hkv][3][BS]
    cache = workloads.pack_tq4(torch.from_numpy(k_idx), torch.from_numpy(v_idx),
                               torch.from_numpy(meta)).numpy()
    cent = np.asarray(_E4M3_EXACT_CENTROIDS, dtype=np.float32)
    q = torch.randn((S, Hkv * QG, D), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    # the equivalent fp8 form: codes of the exact values, scales = norms / V scales
    k_codes = torch.from_numpy(cent[k_idx]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    v_codes = torch.from_numpy(v_idx.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.stack([knorm.astype(np.float32), vscale.astype(np.float32)], axis=2)  # [NB][Hkv][2][BS]
    return dict(q=q_bits, cache=cache, cent=cent, bt=bt, sl=lens, Hkv=Hkv, BS=BS,
                k_codes=k_codes, v_codes=v_codes, scales=np.ascontiguousarray(scales))


def pin_tq4_matches_fp8_form(orc):
    """A 4-bit cache whose dequantized values are all e4m3-exact gives the same bits as the
    fp8 oracle on the fp8 cache holding those values (K codes of centroids[index] with the
    norm as scale, V codes of the index with the V scale as scale): the 4-bit addressing,
    nibble order and field order against the separately pinned fp8 path."""
    for seed in (3, 4):
        p = _tq4_problem(seed)
        a = orc.decode_tq4(p["q"], p["cache"], p["cent"], p["bt"], p["sl"], 0.0883883461356163,
                           p["Hkv"], p["BS"])
        b = orc.decode(p["q"], p["k_codes"], p["v_codes"], p["scales"], p["bt"], p["sl"],
                       0.0883883461356163)
        assert np.array_equal(a, b)
        assert np.abs(a).max() > 0.5


def pin_tq4_constant_v(orc):
    """Every V index 9 with V scale 0.375 and zero point -1.25: every value is 2.125 and so is
    every output row, whatever the K side."""
    p = _tq4_problem(5, v_const=9, v_scale=0.375, v_zero=-1.25)
    out = orc.decode_tq4(p["q"], p["cache"], p["cent"], p["bt"], p["sl"], 0.0883883461356163,
                         p["Hkv"], p["BS"])
    assert np.max(np.abs(out - 2.125)) < 1e-13


ALL_PINS = [pin_e4m3fn_points, pin_e4m3fn_library, pin_bf16_library, pin_dense_bruteforce, pin_sdpa,
            pin_single_token, pin_zero_query, pin_constant_v, pin_two_token_golden,
            pin_block_permutation, pin_split_merge, pin_v_scale_linearity, pin_dominant_token,
            pin_zero_length, pin_e4m3fn_encode_roundtrip, pin_e4m3fn_encode_ties_and_saturation,
            pin_e4m3fn_encode_library, pin_kv_write_quantizer, pin_partials_closed_form, pin_kv_write_matches_library_quantizer,
            pin_f16_library, pin_tq4_golden_record, pin_tq4_matches_fp8_form, pin_tq4_constant_v,
            pin_aliased_blocks, pin_signed_scales, pin_slot_major_transposition,
            pin_two_token_slot_major_golden, pin_tq4_golden_record_slot_major,
            pin_tq4_slot_major_transposition, pin_kv_write_slot_major]
