"""The torch.autograd functions (gated_linear_attention_fwd_amd.autograd) route
to the C-ABI calls: the gradients autograd produces equal, bit for bit, those
of gla_bwd_framecausal / gla_bwd_bidir called directly with the same output
gradients (those calls are checked against the backward oracle in
test_gpu_bwd.py)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
from gated_linear_attention_fwd_amd import autograd as ga
from gated_linear_attention_fwd_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.load_library()
    yield
    torch.cuda.synchronize()


def leaves(B=1, H=3, F=4, T=100, d=64, seed=0, carry=True):
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=seed, scale_qkv=True)
    t = {n: torch.from_numpy(x[n].view(np.int16)).to(DEV).view(torch.bfloat16).requires_grad_()
         for n in "qkvg"}
    t["gamma"] = torch.from_numpy(x["gamma"]).to(DEV).requires_grad_()
    if carry:
        gen = torch.Generator(device=DEV)
        gen.manual_seed(seed + 1)
        t["S_in"] = torch.randn((B, H, d, d), generator=gen, device=DEV).requires_grad_()
        t["z_in"] = torch.rand((B, H, d), generator=gen, device=DEV).requires_grad_()
    return t


@pytest.mark.parametrize("save_states", [True, False])
@pytest.mark.parametrize("use_state_out", [True, False])
def test_framecausal_grads_equal_direct_backward(save_states, use_state_out):
    t = leaves(seed=3)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    w = torch.randn(t["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    wS = torch.randn(t["S_in"].shape, generator=gen, device=DEV)
    wz = torch.randn(t["z_in"].shape, generator=gen, device=DEV)
    o, S, z = ga.gla_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S_in"],
                                 t["z_in"], save_states=save_states, return_state=True)
    loss = (o.float() * w.float()).sum()
    if use_state_out:
        loss = loss + (S * wS).sum() + (z * wz).sum()
    names = ["q", "k", "v", "g", "gamma", "S_in", "z_in"]
    got = dict(zip(names, torch.autograd.grad(loss, [t[n] for n in names])))
    want = gla.gla_bwd_framecausal(
        *(t[n].detach() for n in ("q", "k", "v", "g", "gamma")), w,
        S_in=t["S_in"].detach(), z_in=t["z_in"].detach(),
        dS_out=wS if use_state_out else None, dz_out=wz if use_state_out else None,
        need_state_grad=True)
    for n, m in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("gamma", "dgamma"),
                 ("S_in", "dS_in"), ("z_in", "dz_in")):
        assert torch.equal(got[n], want[m]), n


def test_framecausal_without_carry():
    t = leaves(seed=5, carry=False)
    o = ga.gla_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"])
    w = torch.ones_like(o)
    got = torch.autograd.grad((o.float() * w.float()).sum(), [t["q"], t["k"], t["gamma"]])
    want = gla.gla_bwd_framecausal(*(t[n].detach() for n in ("q", "k", "v", "g", "gamma")), w)
    assert torch.equal(got[0], want["dq"]) and torch.equal(got[1], want["dk"])
    assert torch.equal(got[2], want["dgamma"])


def test_bidir_grads_equal_direct_backward():
    t = leaves(seed=7, F=1, T=300, carry=False)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    w = torch.randn(t["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    o = ga.gla_bidir(t["q"], t["k"], t["v"], t["g"])
    got = torch.autograd.grad((o.float() * w.float()).sum(), [t[n] for n in "qkvg"])
    want = gla.gla_bwd_bidir(*(t[n].detach() for n in "qkvg"), w)
    for x, n in zip(got, ("dq", "dk", "dv", "dg")):
        assert torch.equal(x, want[n]), n


def test_framecausal_on_a_fused_projection():
    """q, k, v as slices of one fused [B, N, 3, H, d] leaf: the gradient that
    reaches the fused tensor holds the three gradients, bit for bit those of
    the contiguous call."""
    B, H, F, T, d = 1, 2, 3, 64, 64
    N = F * T
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    qkv = torch.randn((B, N, 3, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    qkv.requires_grad_()
    g = torch.randn((B, H, N, d), generator=gen, device=DEV).to(torch.bfloat16).requires_grad_()
    gamma = torch.sigmoid(torch.randn((B, H, F), generator=gen, device=DEV) + 2)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    o = ga.gla_framecausal(q, k, v, g, gamma)
    w = torch.randn(o.shape, generator=gen, device=DEV).to(torch.bfloat16)
    (dqkv,) = torch.autograd.grad((o.float() * w.float()).sum(), [qkv])
    want = gla.gla_bwd_framecausal(*(x.detach().contiguous() for x in (q, k, v, g)), gamma, w)
    for i, n in enumerate(("dq", "dk", "dv")):
        assert torch.equal(dqkv[:, :, i].transpose(1, 2), want[n]), n


@pytest.mark.parametrize("save_states", [True, False])
def test_framecausal_loss_reducing_the_state(save_states):
    """A loss that reduces the carried state (S_out.sum() + z_out.mean())
    hands the backward expanded gradients with zero strides: they reach the
    call as dense arrays, and the gradients equal the direct call's for
    dS_out = 1 and dz_out = 1 / (B H d)."""
    t = leaves(seed=13)
    o, S, z = ga.gla_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S_in"],
                                 t["z_in"], save_states=save_states, return_state=True)
    loss = o.float().sum() + S.sum() + z.mean()
    names = ["q", "k", "v", "g", "gamma", "S_in", "z_in"]
    got = dict(zip(names, torch.autograd.grad(loss, [t[n] for n in names])))
    dz = torch.full(t["z_in"].shape, 1.0 / t["z_in"].numel(), device=DEV)
    want = gla.gla_bwd_framecausal(
        *(t[n].detach() for n in ("q", "k", "v", "g", "gamma")), torch.ones_like(o),
        S_in=t["S_in"].detach(), z_in=t["z_in"].detach(), dS_out=torch.ones_like(S),
        dz_out=dz, need_state_grad=True)
    for n, m in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("gamma", "dgamma"),
                 ("S_in", "dS_in"), ("z_in", "dz_in")):
        assert torch.equal(got[n], want[m]), n
