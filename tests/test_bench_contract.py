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
    # kv's mix rewrites the same eighth of its buffer on every launch, which
    # the last-level cache may partly hold
    assert 0 < peak["read2_nt_write_eighth_GBps"] < 10000
    for name in ("720p_5s_bidir", "720p_5s_framecausal", "720p_60s_stream_d128"):
        wl = d["workloads"][name]
        assert wl["ms"]["min"] <= wl["ms"]["median"] <= wl["ms"]["max"], name
        assert wl["tokens_per_s"] > 0 and 0 < wl["frac_of_hbm_peak"] < 1, name
        assert wl["parity"]["max_slab_rel_err"] <= wl["parity"]["bar"], name


@pytest.mark.gpu
def test_stream_probes_move_what_they_document():
    """Each bandwidth probe kind writes what gla_stream_probe documents (2 MiB
    buffers): the write kinds piece i as four copies of i, the copies a, the two
    reads plus one write a ^ b, and kv's mix a ^ b into exactly one eighth of
    the 16-byte pieces, the others untouched."""
    import torch
    sys.path.insert(0, ROOT)
    import gated_linear_attention_fwd_amd as gla

    n = 2 << 20
    gen = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    b = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    xor = torch.bitwise_xor(a, b)
    pieces = torch.arange(n // 16, dtype=torch.int32, device="cuda").repeat_interleave(4)
    for kind in gla.PROBE_KINDS:
        out = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
        gla.stream_probe(kind, out, a, b)
        torch.cuda.synchronize()
        if kind.startswith("write"):
            assert torch.equal(out.view(torch.int32), pieces), kind
        elif kind.startswith("copy"):
            assert torch.equal(out, a), kind
        elif kind.startswith("read2_write1"):
            assert torch.equal(out, xor), kind
        elif kind == "read2_nt_write_eighth":
            written = (out.view(-1, 16) != 0x5A).any(dim=1)
            assert int(written.sum()) == n // 16 // 8, int(written.sum())
            assert torch.equal(out.view(-1, 16)[written], xor.view(-1, 16)[written])
        else:
            assert kind in ("read", "read_nt"), kind
