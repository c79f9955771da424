"""GPU parity of the backward pass (gla_bwd_framecausal, gla_bwd_bidir, through
the C ABI) against the fp64 backward oracle (pinned in test_oracle_bwd.py).

Bar: slab-normalised error (gla_testutil.slab_rel_err) of dq, dk, dv, dg at
most 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs with fp32
accumulation; the fp32 outputs dgamma, dS_in, dz_in by max|d| / max|ref| under
the same per-dtype bar.
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


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    h = host(t)
    return oracle.bf16_to_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


def grad_in(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.bf16_bits(x) if dtype == "bf16" else x


def report(name, errs):
    print(name, " ".join("%s=%.3e" % kv for kv in errs.items()), flush=True)


def compare(got, ref, dtype, name):
    errs = {}
    for n in ("dq", "dk", "dv", "dg"):
        errs[n] = slab_rel_err(f64(got[n]), ref[n])
    for n in ("dgamma", "dS_in", "dz_in"):
        if n in got and n in ref:
            errs[n] = max_abs_over_max(got[n].cpu().numpy(), ref[n])
    report(name, errs)
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    return errs


CASES = [
    # (dtype, B, H, d, F, T, carry)
    ("f32", 1, 2, 16, 4, 16, False),
    ("f32", 1, 3, 64, 3, 37, True),
    ("bf16", 1, 4, 64, 5, 256, True),
    ("bf16", 2, 2, 32, 4, 61, True),
    ("bf16", 1, 2, 128, 3, 100, True),
    ("bf16", 1, 3, 16, 6, 33, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-B%dH%d-d%d-F%dT%d-carry%d" % c)
def test_bwd_framecausal(case, path):
    dtype, B, H, d, F, T, carry = case
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=900 + d + T)
    rng = np.random.default_rng(d + T)
    dO = grad_in(rng, (B, H, F * T, d), dtype)
    S_in = z_in = dS_out = dz_out = None
    if carry:
        S_in = rng.standard_normal((B, H, d, d)).astype(np.float32)
        z_in = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
        dS_out = rng.standard_normal((B, H, d, d)).astype(np.float32)
        dz_out = rng.standard_normal((B, H, d)).astype(np.float32)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "g", "gamma")}
    opt = {n: (None if a is None else dev(a)) for n, a in
           (("S_in", S_in), ("z_in", z_in), ("dS_out", dS_out), ("dz_out", dz_out))}
    got = gla.gla_bwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], dev(dO),
                                  need_state_grad=True, **opt)
    ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                          gamma=x["gamma"], S_in=S_in, z_in=z_in, dS_out=dS_out, dz_out=dz_out)
    compare(got, ref, dtype, "bwd framecausal %s %s" % (case, path))


@pytest.mark.parametrize("dtype,d,N", [("f32", 32, 300), ("bf16", 64, 1000), ("bf16", 128, 129),
                                       ("bf16", 16, 77)])
def test_bwd_bidir(dtype, d, N, path):
    B, H = 1, 3
    x = synth.random_inputs(B, H, 1, N, d, dtype, seed=950 + d)
    rng = np.random.default_rng(N)
    dO = grad_in(rng, (B, H, N, d), dtype)
    got = gla.gla_bwd_bidir(*(dev(x[n]) for n in "qkvg"), dev(dO))
    ref = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], dO)
    compare(got, ref, dtype, "bwd bidir %s d=%d N=%d %s" % (dtype, d, N, path))


def test_bwd_two_blocks_chain():
    """Backward of block 2 first (from dS_out), then block 1 with block 2's
    dS_in as its dS_out: the one-shot gradients."""
    B, H, d, F, T = 1, 4, 64, 6, 96
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=3)
    rng = np.random.default_rng(8)
    dO = dev(grad_in(rng, (B, H, F * T, d), "bf16"))
    dS_out = dev(rng.standard_normal((B, H, d, d)).astype(np.float32))
    dz_out = dev(rng.standard_normal((B, H, d)).astype(np.float32))
    q, k, v, g = (dev(x[n]) for n in "qkvg")
    gamma = dev(x["gamma"])
    full = gla.gla_bwd_framecausal(q, k, v, g, gamma, dO, dS_out=dS_out, dz_out=dz_out,
                                   need_state_grad=True)
    F1 = 2
    s1, s2 = slice(0, F1 * T), slice(F1 * T, F * T)
    _, S1, z1 = gla.gla_fwd_framecausal(q[:, :, s1].contiguous(), k[:, :, s1].contiguous(),
                                        v[:, :, s1].contiguous(), g[:, :, s1].contiguous(),
                                        gamma[:, :, :F1].contiguous(), return_state=True)
    b2 = gla.gla_bwd_framecausal(q[:, :, s2].contiguous(), k[:, :, s2].contiguous(),
                                 v[:, :, s2].contiguous(), g[:, :, s2].contiguous(),
                                 gamma[:, :, F1:].contiguous(), dO[:, :, s2].contiguous(),
                                 S_in=S1, z_in=z1, dS_out=dS_out, dz_out=dz_out)
    b1 = gla.gla_bwd_framecausal(q[:, :, s1].contiguous(), k[:, :, s1].contiguous(),
                                 v[:, :, s1].contiguous(), g[:, :, s1].contiguous(),
                                 gamma[:, :, :F1].contiguous(), dO[:, :, s1].contiguous(),
                                 dS_out=b2["dS_in"], dz_out=b2["dz_in"], need_state_grad=True)
    errs = {}
    for n in ("dq", "dk", "dv", "dg"):
        errs[n] = slab_rel_err(f64(torch.cat([b1[n], b2[n]], dim=2)), f64(full[n]))
    errs["dgamma"] = max_abs_over_max(torch.cat([b1["dgamma"], b2["dgamma"]], dim=2).cpu().numpy(),
                                      full["dgamma"].cpu().numpy().astype(np.float64))
    errs["dS_in"] = max_abs_over_max(b1["dS_in"].cpu().numpy(),
                                     full["dS_in"].cpu().numpy().astype(np.float64))
    report("bwd two blocks", errs)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


def test_bwd_deterministic():
    B, H, d, F, T = 1, 4, 64, 4, 200
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=12)
    rng = np.random.default_rng(1)
    args = [dev(x[n]) for n in ("q", "k", "v", "g", "gamma")] + [
        dev(grad_in(rng, (B, H, F * T, d), "bf16"))]
    a = gla.gla_bwd_framecausal(*args)
    b = gla.gla_bwd_framecausal(*args)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_bwd_empty_and_no_frames():
    """F = 0: no tokens, and the state gradient passes straight through."""
    d = 32
    z4 = torch.empty((1, 2, 0, d), dtype=torch.bfloat16, device=DEV)
    gamma = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dS_out = torch.randn((1, 2, d, d), device=DEV)
    dz_out = torch.randn((1, 2, d), device=DEV)
    out = gla.gla_bwd_framecausal(z4, z4, z4, z4, gamma, z4, dS_out=dS_out, dz_out=dz_out)
    assert torch.equal(out["dS_in"], dS_out) and torch.equal(out["dz_in"], dz_out)
    assert out["dq"].numel() == 0 and out["dgamma"].numel() == 0


def test_bwd_720p_60s_sampled_heads():
    """The 720p/60s shape (B=1, H=32, d=64, 241 frames of 920 tokens, bf16);
    two heads against the oracle."""
    w = synth.WORKLOADS[4]
    xd = synth.device_inputs(w, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    dO = torch.randn(xd["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    got = gla.gla_bwd_framecausal(xd["q"], xd["k"], xd["v"], xd["g"], xd["gamma"], dO,
                                  eps=w.eps)
    torch.cuda.synchronize()
    heads = [0, 21]
    sel = lambda t: np.concatenate([host(t[:, h:h + 1]) for h in heads], axis=1)  # noqa: E731
    ref = oracle.backward(oracle.FRAMECAUSAL, sel(xd["q"]), sel(xd["k"]), sel(xd["v"]),
                          sel(xd["g"]), sel(dO), gamma=sel(xd["gamma"]), eps=w.eps)
    mine = {n: torch.cat([got[n][:, h:h + 1] for h in heads], dim=1)
            for n in ("dq", "dk", "dv", "dg", "dgamma")}
    ref = {n: ref[n] for n in mine}
    compare(mine, ref, "bf16", "bwd 720p/60s heads %s" % heads)
