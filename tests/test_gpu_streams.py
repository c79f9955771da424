"""Every entry point launches on the stream it is given: results on a side
stream equal the default stream's bit for bit, calls on two streams at once
are each correct, and the binding's own allocations (workspace, outputs) stay
reserved for a side stream until its kernels end."""
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


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def inputs(F=5, T=200, d=64, seed=3):
    x = synth.random_inputs(1, 4, F, T, d, "bf16", seed=seed, scale_qkv=True)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "g", "gamma")}
    rng = np.random.default_rng(seed)
    t["beta"] = dev((1 / (1 + np.exp(-rng.standard_normal((1, 4, F * T))))).astype(np.float32))
    t["dO"] = dev(synth.bf16_bits(rng.standard_normal((1, 4, F * T, d)).astype(np.float32)))
    t["S"] = dev(rng.standard_normal((1, 4, d, d)).astype(np.float32))
    t["z"] = dev(np.abs(rng.standard_normal((1, 4, d))).astype(np.float32))
    t["states"] = dev(rng.standard_normal((1, 4, F, d * d + d)).astype(np.float32))
    return t


CALLS = {
    "framecausal": lambda t, s: gla.gla_fwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"],
                                                        t["S"], t["z"], return_state=True,
                                                        stream=s),
    "bidir": lambda t, s: gla.gla_fwd_bidir(t["q"], t["k"], t["v"], t["g"], stream=s),
    "state_carry": lambda t, s: gla.gla_state_carry(t["k"], t["v"], t["gamma"], t["S"], t["z"],
                                                    stream=s),
    "framecausal_ex_rope": lambda t, s: gla.gla_fwd_framecausal_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], rope=gla.Rope3D.video(10, 20, 64), stream=s),
    "bwd": lambda t, s: gla.gla_bwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"],
                                                S_in=t["S"], z_in=t["z"], need_state_grad=True,
                                                stream=s),
    "fwd_states": lambda t, s: gla.gla_fwd_framecausal_states(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S"], t["z"], return_state=True, stream=s),
    "bwd_states": lambda t, s: gla.gla_bwd_framecausal_states(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["states"], t["dO"], S_in=t["S"],
        z_in=t["z"], need_state_grad=True, stream=s),
    "fwd_states_ex": lambda t, s: gla.gla_fwd_framecausal_states_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S"], t["z"], return_state=True, stream=s),
    "bwd_ex": lambda t, s: gla.gla_bwd_framecausal_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"], states=None, S_in=t["S"],
        z_in=t["z"], need_state_grad=True, stream=s),
    "bwd_rope": lambda t, s: gla.gla_bwd_framecausal_ex(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"], S_in=t["S"], z_in=t["z"],
        rope=gla.Rope3D.video(10, 20, 64, frame_offset=1), need_state_grad=True, stream=s),
    "gdn": lambda t, s: gla.gla_gdn_framecausal(t["q"], t["k"], t["v"], t["beta"], t["gamma"],
                                                t["S"], return_state=True, stream=s),
    "anchor": lambda t, s: gla.gla_softmax_anchor(t["q"], t["k"], t["v"], t["g"], T=200,
                                                  n_sink=1, window=2, stream=s),
}


def flat(r):
    if isinstance(r, torch.Tensor):
        return [r]
    if isinstance(r, dict):
        return [r[k] for k in sorted(r)]
    return list(r)


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(flat(a), flat(b)))


@pytest.mark.parametrize("name", sorted(CALLS))
def test_side_stream_equals_default_stream(name):
    t = inputs()
    ref = CALLS[name](t, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    got = CALLS[name](t, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert same(got, ref), name


def test_raw_stream_handle():
    """A stream given as its raw handle (as a C caller would)."""
    t = inputs()
    ref = CALLS["framecausal"](t, None)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    got = CALLS["framecausal"](t, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert same(got, ref)


def test_two_streams_at_once():
    """Two problems in flight on two streams, each with its own workspace."""
    ta, tb = inputs(seed=4), inputs(F=3, T=300, seed=5)
    ra, rb = CALLS["framecausal"](ta, None), CALLS["gdn"](tb, None)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        ga = CALLS["framecausal"](ta, s1)
        gb = CALLS["gdn"](tb, s2)
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    assert same(ga, ra) and same(gb, rb)


def test_binding_allocations_stay_reserved_for_the_side_stream():
    """The workspace and outputs the binding allocates on the current stream are
    handed to kernels on a side stream; freeing them at once and filling fresh
    allocations on the current stream must not disturb those kernels."""
    t = inputs(F=8, T=400, seed=6)
    ref = CALLS["framecausal"](t, None)[0].clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        o, _, _ = CALLS["framecausal"](t, side)
        outs.append(o)
        # the call's workspace has been released; the current stream grabs and
        # overwrites memory right away
        junk = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
        junk.fill_(0xFF)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
