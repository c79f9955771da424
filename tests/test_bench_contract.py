"""The benchmark's command-line contract: one JSON line with the agreed keys
(on a GPU), and a clear refusal of more than one GPU (no GPU needed)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_every_committed_traffic_record_names_a_kernel_and_a_workload():
    sys.path.insert(0, ROOT)
    import bench
    import glob
    import re
    n = 0
    for p in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for m in re.finditer(r"<!-- traffic (\{.*?\}) -->", open(p).read()):
            rec = json.loads(m.group(1))
            assert rec["kernel"] and rec["workload"] and rec["bytes_per_launch"] > 0, p
            n += 1
    assert n > 0
    assert bench.source_hash("gla") and bench.source_hash("anchor")


@pytest.mark.gpu
def test_json_line_carries_the_contract_keys():
    r = subprocess.run([sys.executable, BENCH, "--steps", "2", "--warmup", "1", "--no-cpu"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"] == "720p_60s_B1H32d64_F241T920_bf16"
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and 0 < roof["frac"] < 1
    # traffic: the committed counter record when the kernel sources match the
    # profiled build, else null
    assert roof["traffic"] is None or roof["traffic"] > 0
    # per-step spread, the measured ceilings and the other configurations
    st = d["ms_per_step_stats"]
    assert st["min"] <= st["median"] <= st["max"] and st["reps"] == 2
    peak = d["practical_peak"]
    for k in ("read_GBps", "read_nt_GBps", "copy_GBps", "read2_write1_nt_GBps",
              "torch_copy_GBps"):
        assert 0 < peak[k] < 8000, k
    for name in ("720p_5s_bidir", "720p_5s_framecausal", "720p_60s_stream_d128"):
        wl = d["workloads"][name]
        assert wl["ms"]["min"] <= wl["ms"]["median"] <= wl["ms"]["max"], name
        assert wl["tokens_per_s"] > 0 and 0 < wl["frac_of_hbm_peak"] < 1, name
        assert wl["parity"]["max_slab_rel_err"] <= wl["parity"]["bar"], name
