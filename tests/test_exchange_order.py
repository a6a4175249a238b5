"""The release half of the fused kernels' cross-workgroup exchange, checked in the gfx950
assembly the compiler makes from tq_kernels.hip (CPU only: hipcc cross-compiles).

A workgroup stores its partial with device-coherent (sc1) buffer stores, waits until they
have completed (s_waitcnt vmcnt(0)), passes a workgroup barrier, and only then counts itself
in with an atomic add; the last arrival reads every partial.  The source forbids the compiler
to move a memory access across the wait (inline assembly with a memory clobber), and this test
pins the order the compiler emitted: in every instantiation of tq_flat_kernel and
tq_fused_kernel, each arrival count (global_atomic_add) comes after a barrier, which comes
after a vmcnt(0) wait, which comes after the last sc1 store before the count."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    from paged_gqa_decode_amd import build

    out = str(tmp_path_factory.mktemp("asm") / "tq_kernels.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S", "-o", out,
           os.path.join(build.CSRC, "tq_kernels.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    with open(out) as f:
        return f.read()


def kernels(asm: str, name: str):
    """{mangled name: list of instruction lines} for every instantiation of kernel `name`."""
    out = {}
    for m in re.finditer(r"^(_Z\w*" + name + r"\w*):", asm, flags=re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)
        out[m.group(1)] = [ln.strip() for ln in asm[start:end].splitlines()]
    return out


@pytest.mark.parametrize("name", ["tq_flat_kernel", "tq_fused_kernel"])
def test_stores_drained_before_arrival_count(assembly, name):
    found = kernels(assembly, name)
    assert len(found) == 12, sorted(found)  # 3 query group sizes x 2 block sizes x 2 formats
    for kname, lines in found.items():
        idx = lambda pat: [i for i, ln in enumerate(lines) if re.match(pat, ln)]  # noqa: E731
        stores = idx(r"buffer_store\w*\s.*\bsc1\b")
        waits = idx(r"s_waitcnt\s+vmcnt\(0\)")
        barriers = idx(r"s_barrier\b")
        counts = idx(r"global_atomic_add(_u32)?\s")
        assert counts and stores, f"{kname}: no exchange found"
        for a in counts:
            b = max(i for i in barriers if i < a)
            w = max(i for i in waits if i < b)
            st = max(i for i in stores if i < a)
            assert st < w < b < a, (kname, lines[st], lines[w], lines[b], lines[a])
