"""Every entry point can be captured into a HIP graph (no allocation,
synchronisation or memset inside a call) and replayed: each of several replays,
with new inputs copied in and eager work in between, equals an eager call on
the same inputs bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
from gated_linear_attention_fwd_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.load_library()
    yield
    torch.cuda.synchronize()


def draw(seed, F=4, T=150, d=64):
    x = synth.random_inputs(1, 4, F, T, d, "bf16", seed=seed, scale_qkv=True)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)  # noqa: E731
    t = {n: bf(x[n]) for n in "qkvg"}
    rng = np.random.default_rng(seed)
    t["gamma"] = torch.from_numpy(x["gamma"]).to(DEV)
    t["beta"] = torch.from_numpy(
        (1 / (1 + np.exp(-rng.standard_normal((1, 4, F * T))))).astype(np.float32)).to(DEV)
    t["dO"] = bf(synth.bf16_bits(rng.standard_normal((1, 4, F * T, d)).astype(np.float32)))
    t["S"] = torch.from_numpy(rng.standard_normal((1, 4, d, d)).astype(np.float32)).to(DEV)
    t["z"] = torch.from_numpy(np.abs(rng.standard_normal((1, 4, d))).astype(np.float32)).to(DEV)
    t["states"] = torch.from_numpy(
        rng.standard_normal((1, 4, F, d * d + d)).astype(np.float32)).to(DEV)
    return t


CALLS = {
    "framecausal": lambda t: gla.gla_fwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"],
                                                     t["S"], t["z"], return_state=True),
    "bidir": lambda t: gla.gla_fwd_bidir(t["q"], t["k"], t["v"], t["g"]),
    "bwd": lambda t: gla.gla_bwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"],
                                             S_in=t["S"], z_in=t["z"], need_state_grad=True),
    "fwd_states": lambda t: gla.gla_fwd_framecausal_states(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S"], t["z"], return_state=True),
    "bwd_states": lambda t: gla.gla_bwd_framecausal_states(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["states"], t["dO"], S_in=t["S"], z_in=t["z"],
        need_state_grad=True),
    "fwd_states_ex": lambda t: gla.gla_fwd_framecausal_states_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S"], t["z"], return_state=True),
    "bwd_ex": lambda t: gla.gla_bwd_framecausal_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"], states=t["states"], S_in=t["S"],
        z_in=t["z"], need_state_grad=True),
    "bwd_rope": lambda t: gla.gla_bwd_framecausal_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"], S_in=t["S"], z_in=t["z"],
        rope=gla.Rope3D.video(10, 15, 64, frame_offset=2), need_state_grad=True),
    "bidir_bwd_rope": lambda t: gla.gla_bwd_bidir_ex(
        t["q"], t["k"], t["v"], t["g"], t["dO"], rope=gla.Rope3D.video(10, 15, 64)),
    "gdn": lambda t: gla.gla_gdn_framecausal(t["q"], t["k"], t["v"], t["beta"], t["gamma"],
                                             t["S"], return_state=True),
    "anchor": lambda t: gla.gla_softmax_anchor(t["q"], t["k"], t["v"], t["g"], T=150, n_sink=1,
                                               window=2),
}


def flat(r):
    if isinstance(r, torch.Tensor):
        return [r]
    if isinstance(r, dict):
        return [r[k] for k in sorted(r)]
    return list(r)


@pytest.mark.parametrize("name", sorted(CALLS))
def test_graph_replays_equal_eager_calls(name):
    static = draw(seed=20)
    CALLS[name](static)  # warm up outside the capture (library load, first launches)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = flat(CALLS[name](static))
    for rep, seed in enumerate((21, 22, 23)):
        fresh = draw(seed=seed)
        for n, x in fresh.items():
            static[n].copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in out]
        want = flat(CALLS[name](fresh))  # eager, between replays
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), (name, rep)
