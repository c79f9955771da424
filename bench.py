#!/usr/bin/env python3
"""Throughput of the gated linear-attention forward pass on one MI355X.

One step is one complete library call over the whole workload: the per-frame
KV sums, the decayed state scan and the readout with its normalise-and-gate
epilogue. Default workload: the 720p/60s latent-video shape (B=1, H=32, d=64,
241 frames x 920 tokens, bf16, frame-causal, state carried across frames).

Prints ONE JSON line with tokens/s, the roofline of the dominant kernel
(measured with HIP events inside the timed work's stream), the whole call's
fraction of the HBM roofline, and the fp64 CPU oracle timed on a bounded sample
of the same workload on this host.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GLA fwd tokens/s at 720p/60s shape; % HBM/MFMA roofline vs CPU oracle"
METRIC_BWD = "GLA bwd tokens/s at 720p/60s shape; % HBM/MFMA roofline vs CPU oracle"
METRIC_GDN = "Gated DeltaNet fwd tokens/s at 720p/60s shape; % HBM roofline vs CPU oracle"
METRIC_ANCHOR = ("Gated softmax anchor fwd tokens/s at 720p/60s shape (sink frames + local "
                 "window); % bf16 MFMA roofline vs CPU oracle")
HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
BF16_MFMA_PEAK = 2.5e15  # dense bf16 (and fp16) matrix-core peak, flop/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[2, 3, 4, 5],
                    help="2 small, 3 720p/5s, 4 720p/60s (default), 5 streamed 8 blocks")
    ap.add_argument("--mode", default="framecausal", choices=["framecausal", "bidir"])
    ap.add_argument("--layout", default="bhnd", choices=["bhnd", "fused"],
                    help="bhnd: contiguous [B,H,N,d] tensors; fused: q, k, v as slices of one "
                         "[B,N,3,H,d] projection, g and o [B,N,H,d] (the *_ex entry points)")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="fwd: the forward call (the headline); bwd: the backward call "
                         "(gradients of the forward for a random dL/do)")
    ap.add_argument("--saved-states", action="store_true",
                    help="--pass fwd: the forward that records every frame's state "
                         "(gla_fwd_framecausal_states); --pass bwd: the backward given that "
                         "record (no recompute of the states)")
    ap.add_argument("--mixer", default="gla", choices=["gla", "gdn", "anchor"],
                    help="gla: gated linear attention (the headline); gdn: the frame-wise "
                         "Gated DeltaNet (beta = sigmoid of a normal draw per token); anchor: "
                         "the gated softmax anchor (frame-causal with --sink and --window, "
                         "or over every key with --mode bidir)")
    ap.add_argument("--sink", type=int, default=1, help="anchor: sink frames")
    ap.add_argument("--window", type=int, default=4,
                    help="anchor: frames in the local window, the query's own included")
    ap.add_argument("--rope", action="store_true",
                    help="fused 3D rotary positions over the latent grid (the *_ex entry points)")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="heads of the workload the CPU oracle runs (0: skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default run only: skip the other workloads (720p/5s in both modes, "
                         "the d = 128 stream) and the practical-peak probes")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


# The sources each family's kernels are built from (besides the shared headers,
# the API file and the build flags): a counter record stays valid while these
# are unchanged.
KERNEL_SOURCES = {
    "gla": ["mfma.hip", "valu.hip", "carry.hip", "rope_tab.hpp"],
    "bwd": ["bwd.hip", "bwd_mfma.hip", "mfma.hip", "valu.hip", "carry.hip", "rope_tab.hpp"],
    "gdn": ["gdn.hip", "gdn_mfma.hip"],
    "anchor": ["anchor.hip"],
}
SHARED_SOURCES = ["common.hpp", "mfma_util.hpp", "plan.hpp", "gla_api.cpp"]


def source_hash(family=None) -> str:
    """Hash of the kernel sources (all of them, or one family's with the shared
    files and the build script)."""
    csrc = os.path.join(ROOT, "gated_linear_attention_fwd_amd", "csrc")
    if family is None:
        paths = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        paths = [os.path.join(csrc, n) for n in sorted(SHARED_SOURCES + KERNEL_SOURCES[family])]
        paths.append(os.path.join(ROOT, "gated_linear_attention_fwd_amd", "build.py"))
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, family: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current sources of the kernel's family; else None."""
    for p in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        txt = open(p).read()
        for m in re.finditer(r"<!-- traffic (\{.*?\}) -->", txt):
            rec = json.loads(m.group(1))
            if (rec.get("kernel") == kernel and rec.get("workload") == workload
                    and rec.get("source_hash") == source_hash(family)):
                return rec
    return None


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; --gpus %d (WORLD_SIZE=%d) is not "
              "supported. Heads and batch shard across GPUs with no exchange; see the design "
              "notes." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_linear_attention_fwd_amd as gla
    from gated_linear_attention_fwd_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gla.load_library()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    w = synth.WORKLOADS[args.workload]
    mode = args.mode
    if mode not in w.modes and args.workload != 3:
        mode = w.modes[0]
    es = 4 if w.dtype == "f32" else 2
    print("bench: workload %s mode %s, drawing inputs on the device" % (w.name, mode),
          file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- inputs
    if args.workload == 5:
        blocks = [synth.device_inputs(w, dev, block=b) for b in range(len(w.blocks))]
    elif args.workload == 4:
        blocks = [synth.device_inputs(w, dev)]
    else:
        x = synth.workload_inputs(w)
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

        def todev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
            return torch.from_numpy(a).to(dev)
        blocks = [{n: todev(x[n]) for n in ("q", "k", "v", "g", "gamma")}]
    d = w.d
    S = torch.zeros((w.B, w.H, d, d), dtype=torch.float32, device=dev)
    z = torch.zeros((w.B, w.H, d), dtype=torch.float32, device=dev)
    ex = args.layout != "bhnd" or args.rope
    if args.layout == "fused":
        # q, k, v as slices of one [B, N, 3, H, d] projection; g and o [B, N, H, d]
        for b in blocks:
            X = torch.stack([b.pop("q"), b.pop("k"), b.pop("v")], dim=0)
            X = X.permute(1, 3, 0, 2, 4).contiguous()
            b["q"], b["k"], b["v"] = (X[:, :, i].transpose(1, 2) for i in range(3))
            b["g"] = b["g"].transpose(1, 2).contiguous().transpose(1, 2)
        outs = [torch.empty((w.B, b["q"].shape[2], w.H, d), dtype=b["q"].dtype,
                            device=dev).transpose(1, 2) for b in blocks]
    else:
        outs = [torch.empty_like(b["q"]) for b in blocks]
    grid = synth.LATENT_GRID_720P if w.T == synth.LATENT_TOKENS_720P else None
    if args.rope and grid is None:
        print("bench.py: --rope needs the 720p latent grid", file=sys.stderr)
        sys.exit(2)
    bounds = synth.stream_block_bounds(w) if len(blocks) > 1 else [(0, w.F)]
    ropes = [gla.Rope3D.video(grid[0], grid[1], d, frame_offset=f0) if args.rope else None
             for f0, _ in bounds]
    if mode == "bidir":
        wsb = gla.gla_fwd_bidir_ex_workspace(w.B, w.H, w.F, w.T, d, ropes[0])
    else:
        wsb = max(gla.gla_fwd_framecausal_workspace(w.B, w.H, b["gamma"].shape[-1], w.T, d)
                  for b in blocks)
    bwd = args.which == "bwd"
    gdn = args.mixer == "gdn"
    if gdn and (bwd or ex or mode != "framecausal"):
        print("bench.py: the Gated DeltaNet runs frame-causal, forward, contiguous",
              file=sys.stderr)
        sys.exit(2)
    anchor = args.mixer == "anchor"
    if anchor and (bwd or ex or len(blocks) > 1):
        print("bench.py: the anchor runs forward, contiguous, in one call (workloads 2-4)",
              file=sys.stderr)
        sys.exit(2)
    if gdn:
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed * 1000 + 11)
        for b in blocks:
            b["beta"] = torch.sigmoid(torch.randn(b["q"].shape[:3], generator=gen, device=dev))
        wsb = max(gla.gla_gdn_framecausal_workspace(w.B, w.H, b["gamma"].shape[-1], w.T, d)
                  for b in blocks)
    saved = args.saved_states
    if saved and (mode != "framecausal" or args.mixer != "gla"):
        print("bench.py: --saved-states goes with the frame-causal linear mixer",
              file=sys.stderr)
        sys.exit(2)
    if saved and not bwd:
        rec = [torch.empty((w.B, w.H, b["gamma"].shape[-1], d * d + d), dtype=torch.float32,
                           device=dev) for b in blocks]
    if bwd:
        # dL/do drawn on the device; for a stream, the forward states at the block
        # boundaries (the S_in of each block) are computed once, before timing
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed * 1000 + 7)
        for b in blocks:
            b["dO"] = torch.randn(b["q"].shape, generator=gen, device=dev).to(b["q"].dtype)
        grads = [{n: torch.empty_like(b["q"]) for n in ("dq", "dk", "dv", "dg")} for b in blocks]
        for gd, b in zip(grads, blocks):
            gd["dgamma"] = torch.empty_like(b["gamma"])
        s_in = [None] * len(blocks)
        if len(blocks) > 1:
            Sb = torch.zeros_like(S)
            zb = torch.zeros_like(z)
            for i, b in enumerate(blocks):
                s_in[i] = (Sb.clone(), zb.clone())
                _, Sb, zb = gla.gla_fwd_framecausal_ex(b["q"], b["k"], b["v"], b["g"],
                                                       b["gamma"], Sb, zb, eps=w.eps,
                                                       rope=ropes[i], return_state=True)
            for gd in grads:
                gd["dS_in"] = torch.empty_like(S)
                gd["dz_in"] = torch.empty_like(z)
        if saved:  # the forward's record of every frame's state, made before timing
            for b, si, r in zip(blocks, s_in, ropes):
                _, b["states"] = gla.gla_fwd_framecausal_states_ex(
                    b["q"], b["k"], b["v"], b["g"], b["gamma"], si[0] if si else None,
                    si[1] if si else None, eps=w.eps, rope=r)
        if mode == "bidir":
            wsb = gla.gla_bwd_bidir_ex_workspace(w.B, w.H, w.F, w.T, d, ropes[0])
        elif saved:
            wsb = max(gla.gla_bwd_framecausal_states_workspace(
                w.B, w.H, b["gamma"].shape[-1], w.T, d) for b in blocks)
        else:
            wsb = max(gla.gla_bwd_framecausal_workspace(w.B, w.H, b["gamma"].shape[-1], w.T, d)
                      for b in blocks)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def step_bwd():
        if mode == "bidir":
            b = blocks[0]
            if ex:
                gla.gla_bwd_bidir_ex(b["q"], b["k"], b["v"], b["g"], b["dO"], eps=w.eps,
                                     rope=ropes[0], frames=w.F, out=grads[0], workspace=ws)
            else:
                gla.gla_bwd_bidir(b["q"], b["k"], b["v"], b["g"], b["dO"], eps=w.eps,
                                  out=grads[0], workspace=ws)
            return
        dS = dz = None  # the stream's last block first
        for i in reversed(range(len(blocks))):
            b, si = blocks[i], s_in[i]
            kw = dict(S_in=si[0] if si else None, z_in=si[1] if si else None, dS_out=dS,
                      dz_out=dz, eps=w.eps, out=grads[i], workspace=ws)
            if ex:  # views and/or rotary positions
                r = gla.gla_bwd_framecausal_ex(b["q"], b["k"], b["v"], b["g"], b["gamma"],
                                               b["dO"], states=b.get("states"), rope=ropes[i],
                                               **kw)
            elif saved:
                r = gla.gla_bwd_framecausal_states(b["q"], b["k"], b["v"], b["g"], b["gamma"],
                                                   b["states"], b["dO"], **kw)
            else:
                r = gla.gla_bwd_framecausal(b["q"], b["k"], b["v"], b["g"], b["gamma"], b["dO"],
                                            **kw)
            dS, dz = r.get("dS_in"), r.get("dz_in")

    def step_gdn():
        carry = len(blocks) > 1
        if carry:
            S.zero_()
        for b, o in zip(blocks, outs):
            gla.gla_gdn_framecausal(b["q"], b["k"], b["v"], b["beta"], b["gamma"],
                                    S if carry else None, out=o, S_out=S, workspace=ws)

    def step_anchor():
        b = blocks[0]
        gla.gla_softmax_anchor(b["q"], b["k"], b["v"], b["g"], T=w.T,
                               causal=mode == "framecausal", n_sink=args.sink,
                               window=args.window, out=outs[0])

    def step():
        if anchor:
            step_anchor()
            return
        if gdn:
            step_gdn()
            return
        if bwd:
            step_bwd()
            return
        if mode == "bidir":
            b = blocks[0]
            if ex:
                gla.gla_fwd_bidir_ex(b["q"], b["k"], b["v"], b["g"], eps=w.eps, rope=ropes[0],
                                     frames=w.F, out=outs[0], workspace=ws)
            else:
                gla.gla_fwd_bidir(b["q"], b["k"], b["v"], b["g"], eps=w.eps, out=outs[0],
                                  workspace=ws)
            return
        carry = len(blocks) > 1
        if carry:
            S.zero_()
            z.zero_()
        for i, (b, o, r) in enumerate(zip(blocks, outs, ropes)):
            if ex:
                gla.gla_fwd_framecausal_ex(b["q"], b["k"], b["v"], b["g"], b["gamma"],
                                           S if carry else None, z if carry else None,
                                           eps=w.eps, rope=r, out=o, S_out=S, z_out=z,
                                           workspace=ws)
            elif saved:
                gla.gla_fwd_framecausal_states(b["q"], b["k"], b["v"], b["g"], b["gamma"],
                                               S if carry else None, z if carry else None,
                                               eps=w.eps, out=o, states=rec[i],
                                               S_out=S, z_out=z, workspace=ws)
            else:
                gla.gla_fwd_framecausal(b["q"], b["k"], b["v"], b["g"], b["gamma"],
                                        S if carry else None, z if carry else None, eps=w.eps,
                                        out=o, S_out=S, z_out=z, workspace=ws)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    tokens = w.B * w.N
    value = tokens / (ms_per_step / 1e3)

    # ---------------------------------------------------------------- per-kernel times
    launches_per_step = ((4 if saved else 6) if bwd else 3) * len(blocks)
    gla.profile_begin(launches_per_step * args.steps)
    for _ in range(args.steps):
        step()
    prof = gla.profile_end()
    torch.cuda.synchronize()
    # algorithmic bytes per token-head of each kernel
    per_unit = {"kv": 2 * d * es, "readout": 3 * d * es, "carry": 0,
                "bwd_q": 5 * d * es, "bwd_k": 4 * d * es,
                "gdn_kv": 2 * d * es + 4, "gdn_readout": 2 * d * es}
    token_heads = w.B * w.H * w.N
    # anchor: 4 d flops per (query, visible key) pair (scores and P V)
    pairs = anchor_pairs(w, mode == "framecausal", args.sink, args.window) if anchor else 0
    anchor_flops = 4 * d * pairs * w.B * w.H
    kernels = {}
    for name, (n, total) in prof.items():
        avg_ms = total / n
        launches_per_call = n / args.steps
        alg = per_unit.get(name, 0) * token_heads / launches_per_call
        kernels[name] = {"avg_ms": round(avg_ms, 5), "launches_per_step": launches_per_call,
                         "alg_bytes_per_launch": int(alg),
                         "alg_GBps": round(alg / (avg_ms / 1e3) / 1e9, 1) if alg else 0.0}
        if name == "anchor":
            fl = anchor_flops / launches_per_call
            kernels[name]["alg_flops_per_launch"] = int(fl)
            kernels[name]["alg_TFLOPs"] = round(fl / (avg_ms / 1e3) / 1e12, 1)
    dom = max(prof, key=lambda k: prof[k][1])
    dk = kernels[dom]
    achieved = dk["alg_bytes_per_launch"] / (dk["avg_ms"] / 1e3)
    variant = w.name + "/" + mode + ("/fused" if args.layout == "fused" else "") + \
        ("/rope" if args.rope else "") + ("/bwd" if bwd else "") + \
        ("/states" if saved else "") + ("/gdn" if gdn else "") + \
        ("/anchor" if anchor else "")
    family = "anchor" if anchor else ("gdn" if gdn else ("bwd" if bwd else "gla"))
    traffic_rec = committed_traffic(dom, variant, family)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved / 1e9, 1),
                "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                "traffic": traffic_rec["bytes_per_launch"] if traffic_rec else None}
    if anchor:  # dense contractions (scores on bf16, P V on fp16 matrix cores: one 2.5 PFLOP/s peak)
        fl = dk["alg_flops_per_launch"] / (dk["avg_ms"] / 1e3)
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(fl / 1e12, 1),
                    "peak": BF16_MFMA_PEAK / 1e12, "unit": "TFLOP/s",
                    "frac": round(fl / BF16_MFMA_PEAK, 4),
                    "traffic": traffic_rec["bytes_per_launch"] if traffic_rec else None}
    # forward: read q, k, v, g, write o; backward: read q, k, v, g, dO, write dq,
    # dk, dv, dg (the recompute's second read of k and v is not counted; with
    # saved states there is none)
    if anchor:  # read q, k, v, g, write o (re-reads of k and v from cache not counted)
        call_bytes = w.io_bytes()
        flops = anchor_flops
    elif gdn:  # read q, k, v, beta, write o
        call_bytes = w.io_bytes() * 4 // 5 + 4 * token_heads
        flops = 6 * d * d * token_heads  # U, A, readout
    else:
        call_bytes = w.io_bytes() * 9 // 5 if bwd else w.io_bytes()
        flops = (12 if bwd else 4) * d * d * token_heads
    call = {"alg_bytes": call_bytes, "GBps": round(call_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "frac_of_hbm_peak": round(call_bytes / (ms_per_step / 1e3) / HBM_PEAK, 4),
            "flops": flops,
            "frac_of_bf16_mfma_peak": round(flops / (ms_per_step / 1e3) / BF16_MFMA_PEAK, 4)}

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    parity = None
    if not args.no_cpu and args.cpu_heads > 0:
        if anchor:
            cpu, parity = cpu_baseline_anchor(args, w, mode, blocks, outs, value)
        elif gdn:
            cpu, parity = cpu_baseline_gdn(args, w, blocks, outs, value)
        elif bwd:
            cpu, parity = cpu_baseline_bwd(args, w, mode, blocks, grads, value,
                                           ropes[0].as_dict() if args.rope else None)
        else:
            cpu, parity = cpu_baseline(args, w, mode, blocks, outs, value,
                                       ropes[0].as_dict() if args.rope else None)

    line = {
        "metric": METRIC_ANCHOR if anchor else (METRIC_GDN if gdn else (
            METRIC_BWD if bwd else METRIC)), "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded normal draws in the latent-video shape; no dataset)",
        "config": {"workload": w.name, "mode": mode, "B": w.B, "H": w.H, "d": d, "F": w.F,
                   "T": w.T, "N": w.N, "blocks": list(w.blocks) or [w.F], "eps": w.eps,
                   "layout": ("q, k, v slices of [B,N,3,H,d]; g, o [B,N,H,d]"
                              if args.layout == "fused" else "[B,H,N,d] contiguous"),
                   "rope": ropes[0].as_dict() if args.rope else None,
                   "pass": ("backward (dq, dk, dv, dg, dgamma for a random dL/do)" + (
                       ", given the forward's per-frame states" if saved else "")) if bwd
                   else ("forward, recording every frame's state" if saved else "forward"),
                   "mixer": ("frame-wise Gated DeltaNet (block delta rule per frame, key "
                             "scale 1/sqrt(d T))" if gdn else (
                                 "gated softmax anchor (%s)" % (
                                     "every key" if mode == "bidir" else
                                     "%d sink frame(s), window of %d frames" % (
                                         args.sink, args.window)) if anchor
                                 else "gated linear attention"))},
        "roofline": roofline, "call": call, "kernels": kernels, "cpu_baseline": cpu,
        "parity": parity, "wall_s": round(wall, 3), "ms_per_step_stats": stats(step_ms),
        "source_hash": source_hash(),
        "kernel_family": family, "family_source_hash": source_hash(family),
    }
    default_run = (args.workload == 4 and mode == "framecausal" and not bwd and not gdn
                   and not anchor and not ex and not saved)
    if default_run and not args.no_workloads:
        # the headline's inputs are no longer needed: free them first
        del blocks, outs, ws
        torch.cuda.empty_cache()
        line["practical_peak"] = practical_peak(dev)
        line["workloads"] = other_workloads(args, dev)
    print(json.dumps(line), flush=True)


def stats(ms):
    """median, min and max of per-rep milliseconds."""
    import statistics
    return {"median": round(statistics.median(ms), 5), "min": round(min(ms), 5),
            "max": round(max(ms), 5), "reps": len(ms)}


def practical_peak(dev, nbytes=1 << 30, reps=10):
    """Event-timed practical HBM ceilings: the library's streaming probes
    (gla_stream_probe: the 16-byte-per-lane access pattern of the mixer's
    kernels) over 1 GiB buffers, four times the 256 MB last-level cache, plus
    torch's own device copy. GB/s of bytes read plus bytes written, median of
    ``reps`` launches."""
    import torch

    import gated_linear_attention_fwd_amd as gla

    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(2)
    out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    moved = {"read": 1, "read_nt": 1, "write": 1, "write_nt": 1, "copy": 2, "copy_nt": 2,
             "read2_write1": 3, "read2_write1_nt": 3, "read2_nt_write_eighth": 2.125}

    def run(fn):
        for _ in range(2):
            fn()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            evs[2 * r].record()
            fn()
            evs[2 * r + 1].record()
        torch.cuda.synchronize()
        return stats([evs[2 * r].elapsed_time(evs[2 * r + 1]) for r in range(reps)])["median"]

    res = {}
    for kind in gla.PROBE_KINDS:
        ms = run(lambda: gla.stream_probe(kind, out, a, b))
        res[kind + "_GBps"] = round(moved[kind] * nbytes / (ms / 1e3) / 1e9, 1)
    ms = run(lambda: out.copy_(a))
    res["torch_copy_GBps"] = round(2 * nbytes / (ms / 1e3) / 1e9, 1)
    res["bytes"] = nbytes
    res["stat"] = "median of %d event-timed launches; GB/s of bytes read + written" % reps
    del a, b, out
    torch.cuda.empty_cache()
    return res


def sampled_parity(oracle_fn, got, sel_heads):
    """max slab-relative error of the sampled heads of ``got`` against the
    oracle's output for them."""
    import numpy as np

    import oracle

    ref = oracle_fn()
    o64 = oracle.bf16_to_f64(got) if got.dtype == np.uint16 else got.astype(np.float64)
    r2 = ref.reshape(1, len(sel_heads), -1)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
    err = np.abs(o64.reshape(r2.shape) - r2) / np.maximum(np.maximum(np.abs(r2), rms), 1e-300)
    return float(err.max())


def other_workloads(args, dev):
    """The other measured configurations, each as its own library calls on
    device-drawn inputs of its shape: 720p/5s bidirectional and frame-causal
    (396 MB per call: the 256 MB last-level cache is flushed by writing 1 GiB
    before every rep), and the 720p/60s stream at B=2, H=40, d=128 in 8 blocks
    with the state carried (22.7 GB per step). ms median/min/max over reps,
    tokens/s and fraction of the 8 TB/s HBM peak at the median, and parity of
    sampled heads against the fp64 oracle."""
    import numpy as np
    import torch

    import gated_linear_attention_fwd_amd as gla
    import oracle
    from gated_linear_attention_fwd_amd import synth

    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    def timed(step, warmup, reps, flush):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            if flush:
                gla.stream_probe("write", flush_buf)
            evs[2 * r].record()
            step()
            evs[2 * r + 1].record()
        torch.cuda.synchronize()
        return stats([evs[2 * r].elapsed_time(evs[2 * r + 1]) for r in range(reps)])

    def kernel_avgs(step, n):
        gla.profile_begin(64 * n)
        for _ in range(n):
            step()
        prof = gla.profile_end()
        return {k: round(v[1] / v[0], 5) for k, v in prof.items()}

    out = {}
    # ---- 720p/5s, both modes, one call each
    w = synth.WORKLOADS[3]
    x = synth.device_inputs(w, dev)
    o = torch.empty_like(x["q"])
    ws = torch.empty(max(gla.gla_fwd_framecausal_workspace(w.B, w.H, w.F, w.T, w.d),
                         gla.gla_fwd_bidir_workspace(w.B, w.H, w.N, w.d), 1),
                     dtype=torch.uint8, device=dev)
    heads = [0, w.H - 1]
    sel = {n: np.concatenate([host(x[n][:, h:h + 1]) for h in heads], axis=1)
           for n in ("q", "k", "v", "g", "gamma")}
    for mode in ("bidir", "framecausal"):
        if mode == "bidir":
            def step():
                gla.gla_fwd_bidir(x["q"], x["k"], x["v"], x["g"], eps=w.eps, out=o, workspace=ws)
        else:
            def step():
                gla.gla_fwd_framecausal(x["q"], x["k"], x["v"], x["g"], x["gamma"], eps=w.eps,
                                        out=o, workspace=ws)
        st = timed(step, 3, 50, flush=True)
        kern = kernel_avgs(step, 5)
        got = np.concatenate([host(o[:, h:h + 1]) for h in heads], axis=1)
        if mode == "bidir":
            ref_fn = lambda: oracle.recurrent(oracle.BIDIR, sel["q"], sel["k"], sel["v"],  # noqa: E731
                                              sel["g"], eps=w.eps)[0]
        else:
            ref_fn = lambda: oracle.recurrent(oracle.FRAMECAUSAL, sel["q"], sel["k"],  # noqa: E731
                                              sel["v"], sel["g"], sel["gamma"], eps=w.eps)[0]
        err = sampled_parity(ref_fn, got, heads)
        med = st["median"]
        out["720p_5s_" + mode] = {
            "workload": w.name, "mode": mode, "ms": st, "tokens_per_s": round(w.B * w.N / (med / 1e3), 1),
            "alg_bytes": w.io_bytes(), "frac_of_hbm_peak": round(w.io_bytes() / (med / 1e3) / HBM_PEAK, 4),
            "kernels_avg_ms": kern, "mall_flushed": True,
            "parity": {"heads": heads, "max_slab_rel_err": err, "bar": 2e-2}}
    del x, o, ws
    torch.cuda.empty_cache()

    # ---- the d = 128 stream: 8 chained calls with the state carried
    w = synth.WORKLOADS[5]
    blocks = [synth.device_inputs(w, dev, block=b) for b in range(len(w.blocks))]
    outs = [torch.empty_like(b["q"]) for b in blocks]
    S = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    z = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(gla.gla_fwd_framecausal_workspace(w.B, w.H, b["gamma"].shape[-1], w.T,
                                                          w.d) for b in blocks),
                     dtype=torch.uint8, device=dev)

    def step():
        S.zero_()
        z.zero_()
        for b, o in zip(blocks, outs):
            gla.gla_fwd_framecausal(b["q"], b["k"], b["v"], b["g"], b["gamma"], S, z, eps=w.eps,
                                    out=o, S_out=S, z_out=z, workspace=ws)

    st = timed(step, 3, 10, flush=False)
    kern = kernel_avgs(step, 2)
    slabs = [(0, 0), (w.B - 1, w.H - 1)]

    def sel_stream(ts):
        return np.concatenate([np.concatenate([host(t[b:b + 1, h:h + 1]) for t in ts], axis=2)
                               for b, h in slabs], axis=1)

    xs = {n: sel_stream([b[n] for b in blocks]) for n in ("q", "k", "v", "g", "gamma")}
    got = sel_stream(outs)
    err = sampled_parity(lambda: oracle.recurrent(oracle.FRAMECAUSAL, xs["q"], xs["k"], xs["v"],
                                                  xs["g"], xs["gamma"], eps=w.eps)[0], got, slabs)
    med = st["median"]
    out["720p_60s_stream_d128"] = {
        "workload": w.name, "mode": "framecausal, %d chained calls (block KV cache)" % len(blocks),
        "ms": st, "tokens_per_s": round(w.B * w.N / (med / 1e3), 1), "alg_bytes": w.io_bytes(),
        "frac_of_hbm_peak": round(w.io_bytes() / (med / 1e3) / HBM_PEAK, 4),
        "kernels_avg_ms": kern, "mall_flushed": False,
        "parity": {"slabs": slabs, "max_slab_rel_err": err, "bar": 2e-2}}
    del blocks, outs, ws, flush_buf
    torch.cuda.empty_cache()
    return out


def cpu_baseline(args, w, mode, blocks, outs, gpu_value, rope=None):
    """Time the fp64 oracle (recurrent form, with rotary positions if rope) on a
    bounded sample of heads of the same workload, scale to tokens/s of the whole
    workload, and check the GPU output of those heads against it."""
    import numpy as np
    import torch

    import oracle

    nh = min(args.cpu_heads, w.B * w.H)
    heads = [(i // w.H, i % w.H) for i in range(nh)]

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    def sel(t):  # the sampled heads, as a [1, nh, ...] array
        return np.concatenate([host(t[b:b + 1, h:h + 1]) for (b, h) in heads], axis=1)

    x = {n: np.concatenate([sel(b[n]) for b in blocks], axis=2) for n in "qkvg"}
    gamma = np.concatenate([sel(b["gamma"]) for b in blocks], axis=2)
    got = np.concatenate([sel(o) for o in outs], axis=2)
    threads = oracle.max_threads()
    ntask = nh * ((w.d + 7) // 8)
    print("bench: CPU oracle on %d heads, %d threads" % (nh, min(threads, ntask)),
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    if rope is not None:
        # the whole stream from frame 0 (each block passed its first frame as offset)
        r0 = dict(rope, frame_offset=0)
        if mode == "bidir":
            ref, _, _ = oracle.rope_recurrent(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"],
                                              F=w.F, T=w.T, eps=w.eps, rope=r0)
        else:
            ref, _, _ = oracle.rope_recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"],
                                              x["g"], gamma, eps=w.eps, rope=r0)
    elif mode == "bidir":
        ref, _, _ = oracle.recurrent(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], eps=w.eps)
    else:
        ref, _, _ = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], gamma,
                                     eps=w.eps)
    el = time.perf_counter() - t0
    # the whole workload is B*H*N head-tokens for B*N tokens
    cpu_tokens_per_s = nh * w.N / el / w.H
    cpu = {"value": round(cpu_tokens_per_s, 1), "unit": "tokens/s",
           "cores": int(min(threads, ntask)), "kind": "oracle",
           "sample": "%d of %d heads (all %d tokens each), recurrent fp64 form%s, %.1f s; "
                     "tokens/s = head-tokens/s / H" % (nh, w.B * w.H, w.N,
                                                       " with rotary positions" if rope else "",
                                                       el),
           "host_cpu": host_cpu_model(), "gpu_over_cpu": round(gpu_value / cpu_tokens_per_s, 1)}
    o64 = oracle.bf16_to_f64(got) if got.dtype == np.uint16 else got.astype(np.float64)
    r2 = ref.reshape(1, nh, -1)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
    err = np.abs(o64.reshape(r2.shape) - r2) / np.maximum(np.maximum(np.abs(r2), rms), 1e-300)
    parity = {"heads": nh, "max_slab_rel_err": float(err.max()),
              "bar": 1e-4 if w.dtype == "f32" else 2e-2}
    return cpu, parity


def anchor_visible_frames(F, f, causal, n_sink, window):
    """Key frames query frame f sees (full mode: all F)."""
    if not causal:
        return F
    lo = 0 if window <= 0 else max(0, f - window + 1)
    return len(set(range(min(n_sink, f + 1))) | set(range(lo, f + 1)))


def anchor_pairs(w, causal, n_sink, window):
    """(query, visible key) pairs of one slab."""
    return sum(w.T * w.T * anchor_visible_frames(w.F, f, causal, n_sink, window)
               for f in range(w.F))


def cpu_baseline_anchor(args, w, mode, blocks, outs, gpu_value):
    """Time oracle.softmax_anchor on a bounded sample -- a few heads, the last
    query frames (each a streaming call over the frames up to it; full mode:
    one frame of queries over every key) -- and check o there."""
    import numpy as np
    import torch

    import oracle

    causal = mode == "framecausal"
    nh = min(args.cpu_heads, 4, w.B * w.H)
    nf = min(w.F, 4 if causal else 1)
    heads = [(i // w.H, i % w.H) for i in range(nh)]

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    def sel(t, rows):
        return np.concatenate([host(t[b:b + 1, h:h + 1, rows]) for (b, h) in heads], axis=1)

    b0, T = blocks[0], w.T
    frames = list(range(w.F - nf, w.F))
    threads = min(oracle.max_threads(), nh)
    print("bench: CPU anchor oracle on %d heads x %d query frames, %d threads" % (nh, nf, threads),
          file=sys.stderr, flush=True)
    el, pairs, worst = 0.0, 0, 0.0
    for f in frames:
        q_rows = slice(f * T, (f + 1) * T)
        k_rows = slice(0, (f + 1) * T) if causal else slice(0, w.F * T)
        q, g = sel(b0["q"], q_rows), sel(b0["g"], q_rows)
        k, v = sel(b0["k"], k_rows), sel(b0["v"], k_rows)
        t0 = time.perf_counter()
        ref = oracle.softmax_anchor(q, k, v, g, T=T, causal=causal, n_sink=args.sink,
                                    window=args.window)
        el += time.perf_counter() - t0
        pairs += T * T * anchor_visible_frames(w.F, f, causal, args.sink, args.window)
        got = sel(outs[0], q_rows)
        o64 = oracle.bf16_to_f64(got) if got.dtype == np.uint16 else got.astype(np.float64)
        r2 = ref.reshape(1, nh, -1)
        rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
        err = np.abs(o64.reshape(r2.shape) - r2) / np.maximum(np.maximum(np.abs(r2), rms), 1e-300)
        worst = max(worst, float(err.max()))
    # scaled by work: the whole call's (query, key) pairs over the sample's
    total_pairs = anchor_pairs(w, causal, args.sink, args.window) * w.B * w.H
    call_s = el * total_pairs / (pairs * nh)
    cpu_tokens_per_s = w.B * w.N / call_s
    cpu = {"value": round(cpu_tokens_per_s, 1), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": "%d of %d heads x the last %d query frames (%d tokens each), fp64 softmax "
                     "anchor oracle, %.1f s; scaled to the call by (query, key) pairs"
                     % (nh, w.B * w.H, nf, T, el),
           "host_cpu": host_cpu_model(), "gpu_over_cpu": round(gpu_value / cpu_tokens_per_s, 1)}
    parity = {"heads": nh, "frames": frames, "max_slab_rel_err": worst,
              "bar": 1e-4 if w.dtype == "f32" else 2e-2}
    return cpu, parity


def cpu_baseline_gdn(args, w, blocks, outs, gpu_value):
    """Time oracle.gdn on a bounded sample of heads (the whole stream at once)
    and check o of those heads."""
    import numpy as np
    import torch

    import oracle

    nh = min(args.cpu_heads, w.B * w.H)
    heads = [(i // w.H, i % w.H) for i in range(nh)]

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    def sel(t):
        return np.concatenate([host(t[b:b + 1, h:h + 1]) for (b, h) in heads], axis=1)

    x = {n: np.concatenate([sel(b[n]) for b in blocks], axis=2)
         for n in ("q", "k", "v", "beta", "gamma")}
    got = np.concatenate([sel(o) for o in outs], axis=2)
    threads = min(oracle.max_threads(), nh)
    print("bench: CPU Gated DeltaNet oracle on %d heads, %d threads" % (nh, threads),
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ref, _ = oracle.gdn(x["q"], x["k"], x["v"], x["beta"], x["gamma"],
                        key_scale=1.0 / np.sqrt(w.d * w.T))
    el = time.perf_counter() - t0
    cpu_tokens_per_s = nh * w.N / el / w.H
    cpu = {"value": round(cpu_tokens_per_s, 1), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": "%d of %d heads (all %d tokens each), fp64 Gated DeltaNet oracle, %.1f s; "
                     "tokens/s = head-tokens/s / H" % (nh, w.B * w.H, w.N, el),
           "host_cpu": host_cpu_model(), "gpu_over_cpu": round(gpu_value / cpu_tokens_per_s, 1)}
    o64 = oracle.bf16_to_f64(got) if got.dtype == np.uint16 else got.astype(np.float64)
    r2 = ref.reshape(1, nh, -1)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
    err = np.abs(o64.reshape(r2.shape) - r2) / np.maximum(np.maximum(np.abs(r2), rms), 1e-300)
    parity = {"heads": nh, "max_slab_rel_err": float(err.max()),
              "bar": 1e-4 if w.dtype == "f32" else 2e-2}
    return cpu, parity


def cpu_baseline_bwd(args, w, mode, blocks, grads, gpu_value, rope=None):
    """Time the fp64 backward oracle (with rotary positions if rope) on a
    bounded sample of heads (the whole stream at once), scale to tokens/s, and
    check dq, dk, dv, dg of those heads."""
    import numpy as np
    import torch

    import oracle

    nh = min(args.cpu_heads, w.B * w.H)
    heads = [(i // w.H, i % w.H) for i in range(nh)]

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.contiguous().cpu().numpy()

    def sel(t):
        return np.concatenate([host(t[b:b + 1, h:h + 1]) for (b, h) in heads], axis=1)

    x = {n: np.concatenate([sel(b[n]) for b in blocks], axis=2) for n in ("q", "k", "v", "g", "dO")}
    gamma = np.concatenate([sel(b["gamma"]) for b in blocks], axis=2)
    threads = min(oracle.max_threads(), nh)
    print("bench: CPU backward oracle on %d heads, %d threads" % (nh, threads), file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    # the whole stream at once: its first frame sits at temporal position 0
    r0 = dict(rope, frame_offset=0) if rope is not None else None
    if mode == "bidir":
        ref = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], x["dO"], eps=w.eps,
                              F=w.F if r0 else None, T=w.T if r0 else None, rope=r0)
    else:
        ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["dO"],
                              gamma=gamma, eps=w.eps, rope=r0)
    el = time.perf_counter() - t0
    cpu_tokens_per_s = nh * w.N / el / w.H
    cpu = {"value": round(cpu_tokens_per_s, 1), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": "%d of %d heads (all %d tokens each), fp64 backward oracle, %.1f s; "
                     "tokens/s = head-tokens/s / H" % (nh, w.B * w.H, w.N, el),
           "host_cpu": host_cpu_model(), "gpu_over_cpu": round(gpu_value / cpu_tokens_per_s, 1)}
    worst = 0.0
    for n in ("dq", "dk", "dv", "dg"):
        got = np.concatenate([sel(gd[n]) for gd in grads], axis=2)
        o64 = oracle.bf16_to_f64(got) if got.dtype == np.uint16 else got.astype(np.float64)
        r2 = ref[n].reshape(1, nh, -1)
        rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
        err = np.abs(o64.reshape(r2.shape) - r2) / np.maximum(np.maximum(np.abs(r2), rms),
                                                               1e-300)
        worst = max(worst, float(err.max()))
    parity = {"heads": nh, "max_slab_rel_err": worst, "over": "dq, dk, dv, dg",
              "bar": 1e-4 if w.dtype == "f32" else 2e-2}
    return cpu, parity


if __name__ == "__main__":
    main()
