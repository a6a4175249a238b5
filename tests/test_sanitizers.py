"""Host code under the address and undefined-behaviour sanitizers (CPU only, g++/gcc).

* The C ABI (tq_api.cpp and the launch planning of tq_plan.cpp), built for the host with the
  kernel launchers replaced by recording stand-ins (tests/sanitize/launch_stubs.cpp), driven
  through every entry point with valid and invalid arguments (tests/sanitize/abi_driver.cpp);
  the fused workspace is real host memory sized by tq_fused_workspace_bytes, so its carving is
  checked against the size the library asked for.
* The oracle (oracle/oracle.c), built with the same sanitizers and run on small inputs through
  every entry point in a child process that preloads the sanitizer runtime.

Any report (heap overflow, use after free, signed overflow, misaligned access, ...) aborts
the program, and the test fails."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_gqa_decode_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                                reason="g++ with the sanitizer runtimes is needed")


def test_c_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", *SAN_FLAGS, "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", SAN,
           os.path.join(CSRC, "tq_api.cpp"), os.path.join(CSRC, "tq_plan.cpp"),
           os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all expectations hold" in res.stdout


def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", *SAN_FLAGS, "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-Wall", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm", "-lpthread"], check=True)
    preload = " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",  # the interpreter's own leaks
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, os.path.join(SAN, "oracle_calls.py"), lib],
                         capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "oracle_calls: done" in res.stdout
