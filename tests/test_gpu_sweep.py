"""A seeded sweep of irregular shapes through every entry-point family, each
against the fp64 oracle: odd head counts, batch above one, token counts that
are not multiples of the tile heights, a frame or a few hundred tokens, every
head dimension, both dtypes and, where they apply, carried states. The shapes
are drawn once from a fixed seed, so the sweep is the same on every run.

Bars as in the per-family tests: slab-normalised error 1e-4 (float32 inputs)
and 2e-2 (bfloat16 inputs) for token outputs, max|d| / max|ref| for states and
fp32 gradients.
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


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 6))
        F = int(rng.integers(1, 9))
        T = int(rng.choice([1, 7, 31, 33, 65, 97, 130, 257, 300]))
        carry = bool(rng.random() < 0.5)
        cases.append((i, dtype, B, H, d, F, T, carry))
    return cases


CASES = draw_cases(16, seed=2026)


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def ident(c):
    return "c%d-%s-B%dH%d-d%d-F%dT%d-carry%d" % c


def check(errs, dtype, what):
    print(what, " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], (what, n, e)


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_linear_mixer_forward_backward(case):
    i, dtype, B, H, d, F, T, carry = case
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=3000 + i, scale_qkv=True)
    rng = np.random.default_rng(4000 + i)
    S_in = rng.standard_normal((B, H, d, d)).astype(np.float32) if carry else None
    z_in = np.abs(rng.standard_normal((B, H, d))).astype(np.float32) if carry else None
    t = {n: dev(x[n]) for n in ("q", "k", "v", "g", "gamma")}
    Sd = dev(S_in) if carry else None
    zd = dev(z_in) if carry else None
    # forward, frame-causal, plain and recording the states
    o, S, z = gla.gla_fwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], Sd, zd,
                                      return_state=True)
    o2, states = gla.gla_fwd_framecausal_states(t["q"], t["k"], t["v"], t["g"], t["gamma"], Sd,
                                                zd)
    ro, rS, rz = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                  x["gamma"], S_in, z_in)
    last = states[:, :, -1, :d * d].reshape(B, H, d, d)
    check({"o": slab_rel_err(f64(o), ro), "o_rec": slab_rel_err(f64(o2), ro),
           "S": max_abs_over_max(f64(S), rS), "z": max_abs_over_max(f64(z), rz),
           "S_rec": max_abs_over_max(f64(last), rS)}, dtype, "fwd %s" % (case,))
    # backward, recomputing and from the record
    dO = rng.standard_normal((B, H, F * T, d)).astype(np.float32)
    if dtype == "bf16":
        dO = synth.bf16_bits(dO)
    args = (t["q"], t["k"], t["v"], t["g"], t["gamma"])
    got = gla.gla_bwd_framecausal(*args, dev(dO), S_in=Sd, z_in=zd, need_state_grad=True)
    got2 = gla.gla_bwd_framecausal_states(*args, states, dev(dO), S_in=Sd, z_in=zd,
                                          need_state_grad=True)
    for n in got:
        assert torch.equal(got[n], got2[n]), n
    ref = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                          gamma=x["gamma"], S_in=S_in, z_in=z_in)
    errs = {n: slab_rel_err(f64(got[n]), ref[n]) for n in ("dq", "dk", "dv", "dg")}
    errs.update({n: max_abs_over_max(f64(got[n]), ref[n]) for n in ("dgamma", "dS_in")})
    check(errs, dtype, "bwd %s" % (case,))


@pytest.mark.parametrize("case", CASES[:8], ids=ident)
def test_bidirectional(case):
    i, dtype, B, H, d, F, T, _ = case
    x = synth.random_inputs(B, H, 1, F * T, d, dtype, seed=5000 + i, scale_qkv=True)
    o = gla.gla_fwd_bidir(*(dev(x[n]) for n in "qkvg"))
    ro, _, _ = oracle.recurrent(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"])
    check({"o": slab_rel_err(f64(o), ro)}, dtype, "bidir %s" % (case,))


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_gated_deltanet(case):
    i, dtype, B, H, d, F, T, carry = case
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=6000 + i, scale_qkv=True)
    rng = np.random.default_rng(7000 + i)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, H, F * T))))).astype(np.float32)
    S_in = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32) if carry else None
    o, S = gla.gla_gdn_framecausal(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(beta),
                                   dev(x["gamma"]), dev(S_in) if carry else None,
                                   return_state=True)
    ro, rS = oracle.gdn(x["q"], x["k"], x["v"], beta, x["gamma"], S_in)
    check({"o": slab_rel_err(f64(o), ro), "S": max_abs_over_max(f64(S), rS)}, dtype,
          "gdn %s" % (case,))


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_softmax_anchor(case):
    i, dtype, B, H, d, F, T, carry = case
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=8000 + i, scale_qkv=False)
    rng = np.random.default_rng(9000 + i)
    Fq = int(rng.integers(1, F + 1))
    causal = bool(rng.random() < 0.75)
    n_sink = int(rng.integers(0, 3))
    window = int(rng.integers(0, 4))
    q = x["q"][:, :, (F - Fq) * T:]
    g = x["g"][:, :, (F - Fq) * T:]
    o = gla.gla_softmax_anchor(dev(q), dev(x["k"]), dev(x["v"]), dev(g), T=T, causal=causal,
                               n_sink=n_sink, window=window)
    ro = oracle.softmax_anchor(q, x["k"], x["v"], g, T=T, causal=causal, n_sink=n_sink,
                               window=window)
    check({"o": slab_rel_err(f64(o), ro)}, dtype,
          "anchor %s Fq=%d causal=%d sink=%d window=%d" % (case, Fq, causal, n_sink, window))
