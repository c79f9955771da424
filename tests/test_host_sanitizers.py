"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two programs are built with gcc/g++ and ``-fsanitize=address,undefined
-fno-sanitize-recover=all``, so the first report aborts them:

* the fp64 oracle (``oracle/gla_oracle.c``) with ``host_sanitize/oracle_driver.c``,
  which runs every oracle function on small inputs, empty sizes included, and
  checks the oracle's formulations against one another and its backward pass
  against central differences;
* the C ABI (``gla_api.cpp``: validation, planning, launch sequencing) with
  ``host_sanitize/abi_stubs.cpp`` standing in for the kernel launchers and
  ``host_sanitize/abi_driver.cpp`` calling every entry point. The stand-ins
  touch the first and last element of every range a launch would read or
  write, in host buffers of exactly the documented sizes, so a plan that
  reaches past a workspace or tensor is a heap-buffer-overflow report; the
  driver also checks refused arguments, launch-failure reporting and sizes at
  the limits of the integer types.

Only host code is compiled here (no device code, no GPU needed).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")


def _build(cmd, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path, timeout=300)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr) and "cannot find" in r.stderr:
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr[-300:])
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-4000:]


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:] + "\n" + r.stderr[-6000:])
    assert "0 failures" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is required")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _build(["gcc", "-std=c99", "-fopenmp", *SAN, "-Wall",
            os.path.join(ROOT, "oracle", "gla_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
            "-lm", "-o", exe], tmp_path)
    out = _run(exe)
    assert int(out.split(" checks")[0].split()[-1]) >= 80


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ and the ROCm headers are required")
def test_c_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    _build(["g++", "-std=c++17", *SAN, "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"),
            os.path.join(ROOT, "gated_linear_attention_fwd_amd", "csrc", "gla_api.cpp"),
            os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
            "-o", exe], tmp_path)
    out = _run(exe)
    assert int(out.split(" checks")[0].split()[-1]) >= 200
