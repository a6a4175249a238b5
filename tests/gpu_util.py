"""Helpers shared by the GPU tests: run the HIP path through the binding and
compare with the fp64 oracle."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import paged_gqa_decode_amd as tq
import workloads

MAX_ABS = 1e-2   # bf16 output vs fp64 oracle, every element
MEAN_ABS = 1e-3  # mean over all compared elements
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


PATHS = ("two_kernel", "fused")


def gpu_decode(inp: workloads.Inputs, num_partitions=None, tile_groups=None, partials=None,
               out=None, path="two_kernel"):
    wl = inp.wl
    G = wl.tile_groups_per_partition if tile_groups is None else tile_groups
    P = inp.num_partitions if num_partitions is None else num_partitions
    maxlen = int(inp.seq_lens.max().item())
    res = tq.decode(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, inp.seq_lens,
                    num_partitions=P, tile_groups_per_partition=G,
                    softmax_scale=inp.softmax_scale, max_seq_len=maxlen, partials=partials,
                    out=out, fused=(path == "fused"), kv_layout=inp.kv_layout)
    torch.cuda.synchronize()
    return res


def oracle_decode(inp: workloads.Inputs, units=None):
    c = inp.to("cpu")
    return oracle.decode(c.q, c.k_cache, c.v_cache, c.kv_scales, c.block_tables, c.seq_lens,
                         inp.softmax_scale, units=units, nthreads=ORACLE_THREADS,
                         layout=inp.kv_layout)


def compare(got_bf16: torch.Tensor, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = got_bf16.detach().float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: max_abs {mx:.3e} mean_abs {mean:.3e} (|ref| max {np.abs(ref).max():.3f})")
    assert mx <= max_abs, f"{what}: max abs err {mx:.3e} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean abs err {mean:.3e} > {mean_abs}"
    return mx, mean


_REFS = {}


def cached_ref(key, compute):
    """The oracle's result for `key`, computed once per test session (the largest, the
    bandwidth workload's 1024 (s, h) units, takes about 10 s on 16 threads)."""
    if key not in _REFS:
        say(f"  oracle: computing the reference for {key}")
        _REFS[key] = compute()
    return _REFS[key]


def units_rows(out: torch.Tensor, units, QG):
    """Rows of a [S][Hkv*QG][D] output for the given (s, h) units -> [n][QG][D]."""
    return torch.stack([out[s, h * QG:(h + 1) * QG] for s, h in units])
