"""GPU parity of the per-frame state record (gla_fwd_framecausal_states,
gla_bwd_framecausal_states, through the C ABI).

- the forward's o against the fp64 oracle (bar as for gla_fwd_framecausal:
  slab-normalised error 1e-4 for float32, 2e-2 for bfloat16 inputs);
- every recorded state S_f, z_f against the oracle's state after frames
  0..f (max |d| / max |ref|, same bar);
- the backward given the record equals gla_bwd_framecausal (which recomputes
  the states) bit for bit, and so the backward oracle as well.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
import oracle
from gated_linear_attention_fwd_amd import synth
from gla_testutil import TOL, max_abs_over_max, slab_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.load_library()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=["auto", "valu"])
def path(request, monkeypatch):
    if request.param == "valu":
        monkeypatch.setenv("GLA_PATH", "valu")
    else:
        monkeypatch.delenv("GLA_PATH", raising=False)
    return request.param


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


CASES = [
    # (dtype, B, H, d, F, T, carry)
    ("f32", 1, 2, 16, 4, 16, False),
    ("f32", 1, 3, 64, 3, 37, True),
    ("bf16", 1, 4, 64, 5, 256, True),
    ("bf16", 2, 2, 32, 4, 61, True),
    ("bf16", 1, 2, 128, 3, 100, True),
    ("bf16", 1, 3, 64, 12, 40, False),  # more frames than a kv group of the plain call
]


def inputs(case):
    dtype, B, H, d, F, T, carry = case
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=700 + d + T)
    rng = np.random.default_rng(3 * d + T)
    x["dO"] = rng.standard_normal((B, H, F * T, d)).astype(np.float32)
    if dtype == "bf16":
        x["dO"] = synth.bf16_bits(x["dO"])
    if carry:
        x["S_in"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        x["z_in"] = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
        x["dS_out"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        x["dz_out"] = rng.standard_normal((B, H, d)).astype(np.float32)
    return x


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-B%dH%d-d%d-F%dT%d-carry%d" % c)
def test_forward_records_every_frame_state(case, path):
    dtype, B, H, d, F, T, carry = case
    x = inputs(case)
    t = {n: dev(a) for n, a in x.items()}
    o, states, S_out, z_out = gla.gla_fwd_framecausal_states(
        t["q"], t["k"], t["v"], t["g"], t["gamma"], t.get("S_in"), t.get("z_in"),
        return_state=True)
    assert states.shape == (B, H, F, d * d + d)
    ref_o, ref_S, ref_z = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                           x["gamma"], x.get("S_in"), x.get("z_in"))
    errs = {"o": slab_rel_err(f64(o), ref_o),
            "S_out": max_abs_over_max(S_out.cpu().numpy(), ref_S),
            "z_out": max_abs_over_max(z_out.cpu().numpy(), ref_z)}
    st = states.cpu().numpy()
    for f in range(F):
        n = (f + 1) * T
        _, Sf, zf = oracle.recurrent(oracle.FRAMECAUSAL, *(x[k][:, :, :n] for k in "qkvg"),
                                     x["gamma"][:, :, :f + 1], x.get("S_in"), x.get("z_in"))
        errs["S_%d" % f] = max_abs_over_max(st[:, :, f, :d * d].reshape(B, H, d, d), Sf)
        errs["z_%d" % f] = max_abs_over_max(st[:, :, f, d * d:], zf)
    # the last record is the state handed out
    assert torch.equal(states[:, :, F - 1, :d * d].reshape(B, H, d, d), S_out)
    assert torch.equal(states[:, :, F - 1, d * d:], z_out)
    print("states", case, path, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-B%dH%d-d%d-F%dT%d-carry%d" % c)
def test_backward_from_states_equals_recompute(case, path):
    dtype = case[0]
    x = inputs(case)
    t = {n: dev(a) for n, a in x.items()}
    opt = {n: t.get(n) for n in ("S_in", "z_in", "dS_out", "dz_out")}
    _, states = gla.gla_fwd_framecausal_states(t["q"], t["k"], t["v"], t["g"], t["gamma"],
                                               opt["S_in"], opt["z_in"])
    args = (t["q"], t["k"], t["v"], t["g"], t["gamma"])
    want = gla.gla_bwd_framecausal(*args, t["dO"], need_state_grad=True, **opt)
    got = gla.gla_bwd_framecausal_states(*args, states, t["dO"], need_state_grad=True, **opt)
    for n in want:
        assert torch.equal(got[n], want[n]), n
    ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["dO"],
                          gamma=x["gamma"], S_in=x.get("S_in"), z_in=x.get("z_in"),
                          dS_out=x.get("dS_out"), dz_out=x.get("dz_out"))
    for n in ("dq", "dk", "dv", "dg"):
        assert slab_rel_err(f64(got[n]), ref[n]) <= TOL[dtype], n
    for n in ("dgamma", "dS_in", "dz_in"):
        assert max_abs_over_max(got[n].cpu().numpy(), ref[n]) <= TOL[dtype], n


def test_no_tokens_records_decayed_carry():
    """T = 0: no tokens, yet every frame still decays the carried state."""
    B, H, d, F = 1, 2, 32, 3
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device=DEV)
    gamma = torch.tensor([[[0.5, 0.25, 2.0]] * H], device=DEV)
    S_in = torch.randn((B, H, d, d), device=DEV)
    z_in = torch.rand((B, H, d), device=DEV)
    o, states = gla.gla_fwd_framecausal_states(e, e, e, e, gamma, S_in, z_in)
    assert o.numel() == 0
    w = torch.cumprod(gamma, dim=-1)  # 0.5, 0.125, 0.25: exact in float32
    for f in range(F):
        wf = w[:, :, f:f + 1]
        assert torch.equal(states[:, :, f, :d * d], S_in.reshape(B, H, d * d) * wf)
        assert torch.equal(states[:, :, f, d * d:], z_in * wf)


def test_720p_60s_backward_from_states_equals_recompute():
    """The 720p/60s shape (B=1, H=32, d=64, 241 frames of 920 tokens, bf16),
    in the launch configuration the benchmark times: the backward given the
    record equals the recomputing backward bit for bit, and the forward's o
    matches gla_fwd_framecausal's within the bf16 bar."""
    w = synth.WORKLOADS[4]
    xd = synth.device_inputs(w, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(78)
    dO = torch.randn(xd["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    args = (xd["q"], xd["k"], xd["v"], xd["g"], xd["gamma"])
    o, states = gla.gla_fwd_framecausal_states(*args, eps=w.eps)
    o_plain = gla.gla_fwd_framecausal(*args, eps=w.eps)
    want = gla.gla_bwd_framecausal(*args, dO, eps=w.eps)
    got = gla.gla_bwd_framecausal_states(*args, states, dO, eps=w.eps)
    torch.cuda.synchronize()
    for n in want:
        assert torch.equal(got[n], want[n]), n
    assert slab_rel_err(f64(o[:, :4]), f64(o_plain[:, :4])) <= TOL["bf16"]


@pytest.mark.parametrize("d", [64, 128])
def test_strided_training_calls_equal_contiguous(d):
    """q, k, v read from a fused [B, N, 3, H, d] projection, g and dO as
    [B, N, H, d] views, gradients written into [B, N, H, d] views: the same
    bits as the contiguous calls on copies, with and without the record."""
    B, H, F, T = 1, 3, 4, 96
    N = F * T
    gen = torch.Generator(device=DEV)
    gen.manual_seed(d)
    qkv = torch.randn((B, N, 3, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    gbnhd = torch.randn((B, N, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    dobnhd = torch.randn((B, N, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    gamma = torch.sigmoid(torch.randn((B, H, F), generator=gen, device=DEV) + 2)
    S_in = torch.randn((B, H, d, d), generator=gen, device=DEV)
    z_in = torch.rand((B, H, d), generator=gen, device=DEV)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    g, dO = gbnhd.transpose(1, 2), dobnhd.transpose(1, 2)
    cq, ck, cv, cg, cdO = (x.contiguous() for x in (q, k, v, g, dO))

    o, st = gla.gla_fwd_framecausal_states_ex(q, k, v, g, gamma, S_in, z_in)
    o_ref, st_ref = gla.gla_fwd_framecausal_states(cq, ck, cv, cg, gamma, S_in, z_in)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)

    outs = {n: torch.empty((B, N, H, d), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
            for n in ("dq", "dk", "dv", "dg")}
    for states in (st, None):
        got = gla.gla_bwd_framecausal_ex(q, k, v, g, gamma, dO, states=states, S_in=S_in,
                                         z_in=z_in, need_state_grad=True, out=dict(outs))
        if states is None:
            want = gla.gla_bwd_framecausal(cq, ck, cv, cg, gamma, cdO, S_in=S_in, z_in=z_in,
                                           need_state_grad=True)
        else:
            want = gla.gla_bwd_framecausal_states(cq, ck, cv, cg, gamma, st_ref, cdO, S_in=S_in,
                                                  z_in=z_in, need_state_grad=True)
        for n in want:
            assert torch.equal(got[n], want[n]), (n, states is None)
