"""The input generator's counter-based random numbers (CPU): splitmix64 against its published
first outputs, the int64 tensor path against plain integer arithmetic, counter addressing
(any slice of a stream equals the same numbers drawn whole), and the distributions the
workloads draw (uniforms, Box-Muller normals, permutations, lengths)."""

import json
import os

import numpy as np
import torch

import workloads as w

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U64 = (1 << 64) - 1


def test_splitmix64_published_outputs():
    with open(os.path.join(GOLDEN, "splitmix64_seed0.json")) as f:
        g = json.load(f)
    assert int(g["gamma"], 16) == w.SPLITMIX_GAMMA
    want = [int(x, 16) for x in g["outputs"]]
    assert [int(x) & U64 for x in w.random_bits(0, 0, len(want), "cpu")] == want
    assert [w.mix64_int((i + 1) * w.SPLITMIX_GAMMA) for i in range(len(want))] == want


def test_tensor_path_matches_integers():
    key = w.stream_key(0x5EED0004, "k")
    for start in (0, 12345, (1 << 40) - 7):
        got = w.random_bits(key, start, 64, "cpu")
        want = [w.mix64_int(key + (start + i + 1) * w.SPLITMIX_GAMMA) for i in range(64)]
        assert [int(x) & U64 for x in got] == want


def test_counter_addressing():
    key = w.stream_key(7, "v")
    whole = w.random_normal(key, 0, 5000, "cpu")
    assert torch.equal(w.random_normal(key, 1234, 777, "cpu"), whole[1234:2011])
    assert not torch.equal(w.random_normal(w.stream_key(7, "k"), 0, 100, "cpu"), whole[:100])


def test_distributions():
    u = w.random_uniform(w.stream_key(1, "q"), 0, 1 << 20, "cpu")
    assert 0.0 < float(u.min()) and float(u.max()) < 1.0
    assert abs(float(u.mean()) - 0.5) < 2e-3
    x = w.random_normal(w.stream_key(2, "q"), 0, 1 << 20, "cpu")
    assert abs(float(x.mean())) < 5e-3 and abs(float(x.std()) - 1.0) < 5e-3
    assert abs(float((x ** 4).mean()) - 3.0) < 0.05
    assert abs(float((x.abs() < 1.0).double().mean()) - 0.682689492) < 2e-3
    p = w.random_permutation(w.stream_key(3, "pool"), 10000)
    assert torch.equal(torch.sort(p).values, torch.arange(10000))
    wl = w.WORKLOADS["w3_s64_ragged"]
    lens = w.draw_seq_lens(wl)
    assert lens.min() >= wl.seq_len_lo and lens.max() <= wl.seq_len_hi and len(set(lens)) > 50
