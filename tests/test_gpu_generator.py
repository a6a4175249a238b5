"""The input generator on the GPU draws the same 64-bit numbers as on the CPU, and normals
that agree to fp64 rounding (the log / cos of the two devices may differ in the last bit).
Needs an MI355X."""

import pytest
import torch

import workloads as w
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_same_numbers_on_both_devices():
    key = w.stream_key(0x5EED0004, "k")
    say("[generator] 2^22 numbers on cuda and cpu")
    a = w.random_bits(key, 1 << 30, 1 << 22, "cuda").cpu()
    b = w.random_bits(key, 1 << 30, 1 << 22, "cpu")
    assert torch.equal(a, b)
    x = w.random_normal(key, 1 << 30, 1 << 22, "cuda").cpu()
    y = w.random_normal(key, 1 << 30, 1 << 22, "cpu")
    assert float((x - y).abs().max()) <= 1e-13
