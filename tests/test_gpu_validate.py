"""TQ_VALIDATE=1: the debug check kernel reports, by device printf, a length above
max_seq_len and a block-table entry outside the pool for a token below the length, on
both decode paths and both formats' entry points; the decode itself still runs
(clamped).  Without the variable nothing is printed.  Needs an MI355X."""

import pytest
import torch

import paged_gqa_decode_amd as tq
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu


def _inputs():
    wl = workloads.small_workload(name="validate", num_seqs=3, num_kv_heads=2,
                                  query_group_size=8, kv_block_size=16, seq_lens=(40, 100, 7),
                                  seed=77)
    return workloads.make_inputs(wl, device="cuda", seq_lens=(40, 100, 7))


def _corrupt(inp):
    bt = inp.block_tables.clone()
    bt[1, 2] = inp.num_blocks + 5    # tokens 32..47 of sequence 1 (length 100)
    bt[0, 5] = -7                    # past ceil(40 / 16) = 3 entries: never read, not reported
    lens = inp.seq_lens.clone()
    lens[2] = 10_000                 # above max_seq_len = 100
    return bt, lens


def test_validate_reports_contract_violations(capfd, monkeypatch):
    inp = _inputs()
    bt, lens = _corrupt(inp)
    monkeypatch.setenv("TQ_VALIDATE", "1")
    for fused in (False, True):
        say(f"[validate] fused={fused}")
        out = tq.decode(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, bt, lens,
                        max_seq_len=100, fused=fused)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
    text = capfd.readouterr().out
    assert text.count(f"tq_validate: block_tables[1][2] = {inp.num_blocks + 5}") == 2, text
    assert text.count("tq_validate: seq_lens[2] = 10000 is outside [0, 100]") == 2, text
    assert "block_tables[0]" not in text, text


def test_validate_is_off_by_default(capfd, monkeypatch):
    inp = _inputs()
    bt, lens = _corrupt(inp)
    monkeypatch.delenv("TQ_VALIDATE", raising=False)
    tq.decode(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, bt, lens, max_seq_len=100,
              fused=True)
    torch.cuda.synchronize()
    assert "tq_validate" not in capfd.readouterr().out


def test_validate_clean_inputs_print_nothing(capfd, monkeypatch):
    inp = _inputs()
    monkeypatch.setenv("TQ_VALIDATE", "1")
    tq.decode(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, inp.seq_lens,
              max_seq_len=100)
    torch.cuda.synchronize()
    assert "tq_validate" not in capfd.readouterr().out
