"""GPU parity of the backward with 3D rotary positions (gla_bwd_framecausal_ex,
gla_bwd_bidir_ex and gla_fwd_framecausal_states_ex with rope, through the C
ABI) against the fp64 backward oracle with the same rotation
(oracle.backward(..., rope=...), pinned by finite differences of the rotary
forward oracle in test_oracle_rope_bwd.py).

Bar as for the backward without positions: slab-normalised error 1e-4 for
float32 and 2e-2 for bfloat16 inputs on the token gradients, max|d| / max|ref|
on the fp32 ones (dgamma, dS_in, dz_in). The backward given the state record
must equal the recomputing one bit for bit; the autograd functions must give
the direct calls' bits.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
import oracle
from gated_linear_attention_fwd_amd import autograd as ga
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
    return t.detach().contiguous().cpu().numpy().astype(np.float64)


def rope_for(gh, gw, d, frame_offset=0, theta=10000.0):
    s = 2 * (d // 6)
    return dict(grid_h=gh, grid_w=gw, frame_offset=frame_offset, dim_t=d - 2 * s, dim_h=s,
                dim_w=s, theta=theta)


def check(errs, dtype, what):
    print(what, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], (what, n, e)


CASES = [
    # (dtype, B, H, d, F, gh, gw, frame_offset, carry)
    ("f32", 1, 2, 16, 3, 3, 5, 0, True),
    ("f32", 1, 2, 32, 4, 4, 9, 5, True),
    ("bf16", 1, 3, 64, 3, 5, 7, 2, True),
    ("bf16", 2, 2, 64, 5, 8, 16, 0, False),
    ("bf16", 1, 2, 128, 3, 6, 11, 7, True),
    ("bf16", 1, 2, 32, 2, 16, 16, 1, True),
    # one token per frame, a temporal position near the 2^30 limit
    ("bf16", 1, 2, 64, 4, 1, 1, (1 << 29) + 3, True),
]


def ident(c):
    return "%s-B%dH%d-d%d-F%d-grid%dx%d-off%d-carry%d" % c


def inputs(case, seed):
    dtype, B, H, d, F, gh, gw, off, carry = case
    T = gh * gw
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=seed, scale_qkv=True)
    rng = np.random.default_rng(seed + 1)
    dO = rng.standard_normal((B, H, F * T, d)).astype(np.float32)
    x["dO"] = synth.bf16_bits(dO) if dtype == "bf16" else dO
    if carry:
        x["S_in"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        x["z_in"] = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
        x["dS_out"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        x["dz_out"] = rng.standard_normal((B, H, d)).astype(np.float32)
    return x, rope_for(gh, gw, d, off)


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_framecausal_backward_matches_oracle(case, path):
    dtype = case[0]
    x, rope = inputs(case, seed=900 + case[3] + case[5])
    t = {n: dev(a) for n, a in x.items()}
    opt = {n: t.get(n) for n in ("S_in", "z_in", "dS_out", "dz_out")}
    args = (t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"])
    got = gla.gla_bwd_framecausal_ex(*args, rope=rope, need_state_grad=True, **opt)
    ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["dO"],
                          gamma=x["gamma"], S_in=x.get("S_in"), z_in=x.get("z_in"),
                          dS_out=x.get("dS_out"), dz_out=x.get("dz_out"), rope=rope)
    errs = {n: slab_rel_err(f64(got[n]), ref[n]) for n in ("dq", "dk", "dv", "dg")}
    errs.update({n: max_abs_over_max(f64(got[n]), ref[n]) for n in ("dgamma", "dS_in", "dz_in")})
    check(errs, dtype, "rope bwd %s %s" % (ident(case), path))
    # the positions matter: the gradients without them are far off
    plain = gla.gla_bwd_framecausal_ex(*args, need_state_grad=True, **opt)
    assert slab_rel_err(f64(plain["dq"]), ref["dq"]) > 10 * TOL[dtype]


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_backward_from_the_rotary_record_equals_recompute(case, path):
    """gla_fwd_framecausal_states_ex with rope: o and the last recorded state
    against the rotary forward oracle, and the backward given the record equal
    to the recomputing backward bit for bit."""
    dtype = case[0]
    x, rope = inputs(case, seed=1900 + case[3] + case[5])
    t = {n: dev(a) for n, a in x.items()}
    opt = {n: t.get(n) for n in ("S_in", "z_in", "dS_out", "dz_out")}
    args = (t["q"], t["k"], t["v"], t["g"], t["gamma"])
    o, states = gla.gla_fwd_framecausal_states_ex(*args, opt["S_in"], opt["z_in"], rope=rope)
    ro, rS, rz = oracle.rope_recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                       x["gamma"], x.get("S_in"), x.get("z_in"), rope=rope)
    B, H, F, E = states.shape
    d = x["q"].shape[-1]
    check({"o": slab_rel_err(f64(o), ro),
           "S_last": max_abs_over_max(f64(states[:, :, F - 1, :d * d]).reshape(B, H, d, d), rS),
           "z_last": max_abs_over_max(f64(states[:, :, F - 1, d * d:]), rz)},
          dtype, "rope states %s %s" % (ident(case), path))
    want = gla.gla_bwd_framecausal_ex(*args, t["dO"], rope=rope, need_state_grad=True, **opt)
    got = gla.gla_bwd_framecausal_ex(*args, t["dO"], states=states, rope=rope,
                                     need_state_grad=True, **opt)
    for n in want:
        assert torch.equal(got[n], want[n]), n


@pytest.mark.parametrize("case", CASES[:5], ids=ident)
def test_bidirectional_backward_matches_oracle(case, path):
    dtype, B, H, d, F, gh, gw, off, _ = case
    x, rope = inputs(case, seed=2900 + d + gh)
    T = gh * gw
    t = {n: dev(x[n]) for n in ("q", "k", "v", "g", "dO")}
    got = gla.gla_bwd_bidir_ex(t["q"], t["k"], t["v"], t["g"], t["dO"], rope=rope)
    ref = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], x["dO"], F=F, T=T,
                          rope=rope)
    errs = {n: slab_rel_err(f64(got[n]), ref[n]) for n in ("dq", "dk", "dv", "dg")}
    check(errs, dtype, "rope bidir bwd %s %s" % (ident(case), path))
    # without positions the call is gla_bwd_bidir, bit for bit
    plain = gla.gla_bwd_bidir_ex(t["q"], t["k"], t["v"], t["g"], t["dO"])
    direct = gla.gla_bwd_bidir(t["q"], t["k"], t["v"], t["g"], t["dO"])
    for n in direct:
        assert torch.equal(plain[n], direct[n]), n


def test_fused_projection_views_equal_contiguous():
    """q, k, v from a fused [B, N, 3, H, d] projection with rotary positions:
    the gradients written into [B, N, H, d] views are the contiguous call's
    bits."""
    B, H, F, gh, gw, d = 1, 3, 3, 6, 8, 64
    T = gh * gw
    N = F * T
    rope = rope_for(gh, gw, d, 4)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    qkv = torch.randn((B, N, 3, H, d), generator=gen, device=DEV).to(torch.bfloat16)
    g = torch.randn((B, N, H, d), generator=gen, device=DEV).to(torch.bfloat16).transpose(1, 2)
    dO = torch.randn((B, N, H, d), generator=gen, device=DEV).to(torch.bfloat16).transpose(1, 2)
    gamma = torch.sigmoid(torch.randn((B, H, F), generator=gen, device=DEV) + 2)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    cq, ck, cv, cg, cdO = (x.contiguous() for x in (q, k, v, g, dO))
    outs = {n: torch.empty((B, N, H, d), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
            for n in ("dq", "dk", "dv", "dg")}
    got = gla.gla_bwd_framecausal_ex(q, k, v, g, gamma, dO, rope=rope, out=dict(outs))
    want = gla.gla_bwd_framecausal_ex(cq, ck, cv, cg, gamma, cdO, rope=rope)
    for n in want:
        assert torch.equal(got[n], want[n]), n
    gb = gla.gla_bwd_bidir_ex(q, k, v, g, dO, rope=rope, out=dict(outs))
    wb = gla.gla_bwd_bidir_ex(cq, ck, cv, cg, cdO, rope=rope)
    for n in wb:
        assert torch.equal(gb[n], wb[n]), n


@pytest.mark.parametrize("save_states", [True, False])
def test_autograd_with_rotary_positions_equals_direct_calls(save_states):
    B, H, F, gh, gw, d = 1, 2, 3, 5, 8, 64
    T = gh * gw
    rope = rope_for(gh, gw, d, 3)
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=31, scale_qkv=True)
    leaf = {n: dev(x[n]).requires_grad_() for n in "qkvg"}
    leaf["gamma"] = dev(x["gamma"]).requires_grad_()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    leaf["S_in"] = torch.randn((B, H, d, d), generator=gen, device=DEV).requires_grad_()
    leaf["z_in"] = torch.rand((B, H, d), generator=gen, device=DEV).requires_grad_()
    w = torch.randn((B, H, F * T, d), generator=gen, device=DEV).to(torch.bfloat16)
    o = ga.gla_framecausal(leaf["q"], leaf["k"], leaf["v"], leaf["g"], leaf["gamma"],
                           leaf["S_in"], leaf["z_in"], save_states=save_states, rope=rope)
    names = ["q", "k", "v", "g", "gamma", "S_in", "z_in"]
    got = dict(zip(names, torch.autograd.grad((o.float() * w.float()).sum(),
                                              [leaf[n] for n in names])))
    want = gla.gla_bwd_framecausal_ex(*(leaf[n].detach() for n in ("q", "k", "v", "g", "gamma")),
                                      w, S_in=leaf["S_in"].detach(), z_in=leaf["z_in"].detach(),
                                      rope=rope, need_state_grad=True)
    for n, m in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("gamma", "dgamma"),
                 ("S_in", "dS_in"), ("z_in", "dz_in")):
        assert torch.equal(got[n], want[m]), n
    ob = ga.gla_bidir(leaf["q"], leaf["k"], leaf["v"], leaf["g"], rope=rope)
    gb = torch.autograd.grad((ob.float() * w.float()).sum(), [leaf[n] for n in "qkvg"])
    wb = gla.gla_bwd_bidir_ex(*(leaf[n].detach() for n in "qkvg"), w, rope=rope)
    for a, n in zip(gb, ("dq", "dk", "dv", "dg")):
        assert torch.equal(a, wb[n]), n


def draw_sweep(n, seed):
    """Irregular shapes, drawn once from a fixed seed: head dimension, dtype,
    batch, heads, frames, the latent grid (tokens per frame), frame offset,
    carried state."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        cases.append((dtype, int(rng.integers(1, 3)), int(rng.integers(1, 4)), d,
                      int(rng.integers(1, 6)), int(rng.integers(1, 13)), int(rng.integers(1, 23)),
                      int(rng.integers(-3, 9)), bool(rng.random() < 0.5)))
    return cases


@pytest.mark.parametrize("case", draw_sweep(10, seed=909), ids=ident)
def test_sweep_of_irregular_shapes(case):
    """Both modes, against the rotary backward oracle, at the drawn shapes."""
    dtype, B, H, d, F, gh, gw, off, carry = case
    x, rope = inputs(case, seed=3900 + d + gh * gw)
    t = {n: dev(a) for n, a in x.items()}
    opt = {n: t.get(n) for n in ("S_in", "z_in", "dS_out", "dz_out")}
    got = gla.gla_bwd_framecausal_ex(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["dO"],
                                     rope=rope, need_state_grad=True, **opt)
    ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["dO"],
                          gamma=x["gamma"], S_in=x.get("S_in"), z_in=x.get("z_in"),
                          dS_out=x.get("dS_out"), dz_out=x.get("dz_out"), rope=rope)
    errs = {n: slab_rel_err(f64(got[n]), ref[n]) for n in ("dq", "dk", "dv", "dg")}
    errs.update({n: max_abs_over_max(f64(got[n]), ref[n]) for n in ("dgamma", "dS_in", "dz_in")})
    gb = gla.gla_bwd_bidir_ex(t["q"], t["k"], t["v"], t["g"], t["dO"], rope=rope)
    rb = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], x["dO"], F=F, T=gh * gw,
                         rope=rope)
    errs.update({"bidir_" + n: slab_rel_err(f64(gb[n]), rb[n]) for n in ("dq", "dk", "dv", "dg")})
    check(errs, dtype, "rope bwd sweep %s" % ident(case))
