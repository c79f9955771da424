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


@pytest.fixture(scope="module")
def abi_exe(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ and the ROCm headers are required")
    tmp_path = tmp_path_factory.mktemp("abi_san")
    exe = str(tmp_path / "abi_san")
    _build(["g++", "-std=c++17", *SAN, "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"),
            os.path.join(ROOT, "gated_linear_attention_fwd_amd", "csrc", "gla_api.cpp"),
            os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
            "-o", exe], tmp_path)
    return exe


def test_c_abi_host_code_under_address_and_undefined_sanitizers(abi_exe):
    out = _run(abi_exe)
    assert int(out.split(" checks")[0].split()[-1]) >= 200


def test_launch_log(abi_exe):
    """GLA_LOG=1: every call prints its plan (the workgroup geometry) and each
    launch, in order, on stderr; without it nothing is printed."""
    r = subprocess.run([abi_exe], capture_output=True, text=True,
                       env=dict(ENV, GLA_LOG="1"), timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    log = [l for l in r.stderr.splitlines() if l.startswith("gla: ")]
    plans = [l for l in log if not l.startswith("gla: launch ")]
    assert any(l.startswith("gla: forward (frame-causal) path=") and " G=" in l and " R=" in l
               and " kv_wgs=" in l and " readout_wgs=" in l for l in plans), plans[:5]
    assert any(l.startswith("gla: forward (bidirectional) path=") for l in plans)
    assert any(l.startswith("gla: backward (frame-causal") for l in plans)
    assert any(l.startswith("gla: gated deltanet path=") for l in plans)
    assert any(l.startswith("gla: softmax anchor path=") and " tiles=" in l for l in plans)
    launches = [l[len("gla: launch "):] for l in log if l.startswith("gla: launch ")]
    for k in ("kv", "carry", "readout", "bwd_q", "rev_scan", "bwd_k", "gdn_kv", "gdn_scan",
              "gdn_readout", "anchor", "anchor_redo"):
        assert k in launches, k
    # a forward's launches follow its plan line in order: kv, carry, readout
    i = next(n for n, l in enumerate(log) if l.startswith("gla: forward (frame-causal) path="))
    nxt = [l for l in log[i + 1:i + 4]]
    assert nxt[:3] == ["gla: launch kv", "gla: launch carry", "gla: launch readout"], nxt
    quiet = subprocess.run([abi_exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert not any(l.startswith("gla: ") for l in quiet.stderr.splitlines())
