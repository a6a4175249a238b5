"""Build libtqdecode.so (the gfx950 kernels and the C ABI) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtqdecode.so")
SOURCES = [os.path.join(CSRC, "tq_kernels.hip"), os.path.join(CSRC, "tq_api.cpp"),
           os.path.join(CSRC, "tq_plan.cpp")]
PROBE_LIB = os.path.join(PKG, "libtqprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "tq_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: hipcc may otherwise pair fp32 arithmetic into packed
# instructions; the code here never needs them.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc(out: str, sources, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build libtqdecode.so (decode kernels + C ABI) and libtqprobe.so (HBM probes)."""
    _hipcc(PROBE_LIB, PROBE_SOURCES, verbose)
    return _hipcc(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
