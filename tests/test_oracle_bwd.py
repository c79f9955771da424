"""Pins of the fp64 backward oracle (oracle.backward).

The pages state the forward pass only; the backward is its chain rule. These
pins tie it to the forward oracle and to the mathematics, never to its own
formulas:
- central finite differences of L = <dO, o> + <dS_out, S_out> + <dz_out, z_out>
  computed with the forward oracle, for every input element;
- linearity in the incoming gradients;
- the single-token closed form;
- gamma = 0 reduces frame-causal gradients to per-frame bidirectional ones;
- gradients chained through two blocks (dS_in of the second block fed as the
  first block's dS_out) equal the one-shot gradients.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gla_testutil import close


def away_from_kinks(rng, shape, margin=0.2):
    """Normal draws pushed at least `margin` away from 0 (ReLU is smooth there)."""
    x = rng.standard_normal(shape)
    return np.sign(x) * (margin + np.abs(x))


def loss(mode, x, dO, dS_out=None, dz_out=None, eps=1e-6):
    o, S, z = oracle.recurrent(mode, x["q"], x["k"], x["v"], x["g"], x.get("gamma"),
                               S_in=x.get("S_in"), z_in=x.get("z_in"), eps=eps)
    L = float(np.sum(dO * o))
    if dS_out is not None:
        L += float(np.sum(dS_out * S)) + float(np.sum(dz_out * z))
    return L


def finite_differences(mode, x, dO, dS_out=None, dz_out=None, h=1e-6, eps=1e-6):
    grads = {}
    for name, a in x.items():
        gd = np.empty_like(a)
        for idx in np.ndindex(a.shape):
            keep = a[idx]
            a[idx] = keep + h
            lp = loss(mode, x, dO, dS_out, dz_out, eps)
            a[idx] = keep - h
            lm = loss(mode, x, dO, dS_out, dz_out, eps)
            a[idx] = keep
            gd[idx] = (lp - lm) / (2 * h)
        grads[name] = gd
    return grads


def inputs(seed, B, H, F, T, d, causal=True, carry=True):
    rng = np.random.default_rng(seed)
    x = {n: away_from_kinks(rng, (B, H, F * T, d)) for n in "qkv"}
    x["g"] = rng.standard_normal((B, H, F * T, d))
    if causal:
        x["gamma"] = rng.uniform(0.3, 0.95, (B, H, F))
        if carry:
            x["S_in"] = rng.standard_normal((B, H, d, d))
            x["z_in"] = rng.uniform(0.5, 2.0, (B, H, d))
    return x, rng


@pytest.mark.parametrize("carry", [False, True])
def test_framecausal_gradients_match_finite_differences(carry):
    B, H, F, T, d = 1, 2, 3, 2, 3
    x, rng = inputs(11 + carry, B, H, F, T, d, carry=carry)
    dO = rng.standard_normal((B, H, F * T, d))
    dS_out = rng.standard_normal((B, H, d, d)) if carry else None
    dz_out = rng.standard_normal((B, H, d)) if carry else None
    got = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                          gamma=x["gamma"], S_in=x.get("S_in"), z_in=x.get("z_in"),
                          dS_out=dS_out, dz_out=dz_out)
    fd = finite_differences(oracle.FRAMECAUSAL, x, dO, dS_out, dz_out)
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("gamma", "dgamma")]
    if carry:
        pairs += [("S_in", "dS_in"), ("z_in", "dz_in")]
    for a, b in pairs:
        err = np.abs(got[b] - fd[a]).max() / max(np.abs(fd[a]).max(), 1e-12)
        assert err < 1e-6, (a, err)


def test_bidirectional_gradients_match_finite_differences():
    B, H, N, d = 1, 2, 5, 3
    x, rng = inputs(21, B, H, 1, N, d, causal=False)
    dO = rng.standard_normal((B, H, N, d))
    got = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], dO)
    fd = finite_differences(oracle.BIDIR, x, dO)
    for a in "qkvg":
        err = np.abs(got["d" + a] - fd[a]).max() / max(np.abs(fd[a]).max(), 1e-12)
        assert err < 1e-6, (a, err)


def test_linear_in_the_incoming_gradients():
    B, H, F, T, d = 1, 1, 3, 4, 4
    x, rng = inputs(31, B, H, F, T, d)
    args = (x["q"], x["k"], x["v"], x["g"])
    kw = dict(gamma=x["gamma"], S_in=x["S_in"], z_in=x["z_in"])
    d1, d2 = (rng.standard_normal((B, H, F * T, d)) for _ in range(2))
    s1, s2 = (rng.standard_normal((B, H, d, d)) for _ in range(2))
    z1, z2 = (rng.standard_normal((B, H, d)) for _ in range(2))
    a = oracle.backward(oracle.FRAMECAUSAL, *args, d1, dS_out=s1, dz_out=z1, **kw)
    b = oracle.backward(oracle.FRAMECAUSAL, *args, d2, dS_out=s2, dz_out=z2, **kw)
    c = oracle.backward(oracle.FRAMECAUSAL, *args, 2 * d1 - 3 * d2, dS_out=2 * s1 - 3 * s2,
                        dz_out=2 * z1 - 3 * z2, **kw)
    for n in a:
        assert close(c[n], 2 * a[n] - 3 * b[n], 1e-12), n


def test_single_token_closed_form():
    """o = sigma(g) v r with r = a / (a + eps), a = phi(q).phi(k):
    dv = dO sigma r, dg = dO v r sigma (1 - sigma), and with
    c = sum_j dO_j sigma_j v_j eps / (a + eps)^2: dq = [q > 0] phi(k) c,
    dk = [k > 0] phi(q) c."""
    rng = np.random.default_rng(4)
    d, eps = 5, 0.3
    q, k, v, g, dO = (rng.standard_normal((1, 1, 1, d)) for _ in range(5))
    got = oracle.backward(oracle.BIDIR, q, k, v, g, dO, eps=eps)
    fq, fk = np.maximum(q, 0), np.maximum(k, 0)
    a = float(np.sum(fq * fk))
    r = a / (a + eps)
    s = expit(g)
    c = float(np.sum(dO * s * v)) * eps / (a + eps) ** 2
    assert close(got["dv"], dO * s * r, 1e-13)
    assert close(got["dg"], dO * v * r * s * (1 - s), 1e-13)
    assert close(got["dq"], (q > 0) * fk * c, 1e-12)
    assert close(got["dk"], (k > 0) * fq * c, 1e-12)


def test_gamma_zero_makes_frames_independent():
    B, H, F, T, d = 1, 2, 3, 4, 3
    x, rng = inputs(5, B, H, F, T, d, carry=False)
    dO = rng.standard_normal((B, H, F * T, d))
    got = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                          gamma=np.zeros((B, H, F)))
    for f in range(F):
        sl = slice(f * T, (f + 1) * T)
        ref = oracle.backward(oracle.BIDIR, x["q"][:, :, sl], x["k"][:, :, sl],
                              x["v"][:, :, sl], x["g"][:, :, sl], dO[:, :, sl])
        for n in ("dq", "dk", "dv", "dg"):
            assert close(got[n][:, :, sl], ref[n], 1e-12), (f, n)


def test_two_blocks_chain_through_the_carried_state():
    """Block 2 takes block 1's S_out as S_in; its dS_in is block 1's dS_out."""
    B, H, F, T, d = 1, 2, 5, 3, 4
    x, rng = inputs(6, B, H, F, T, d)
    dO = rng.standard_normal((B, H, F * T, d))
    dS_out = rng.standard_normal((B, H, d, d))
    dz_out = rng.standard_normal((B, H, d))
    full = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                           gamma=x["gamma"], S_in=x["S_in"], z_in=x["z_in"], dS_out=dS_out,
                           dz_out=dz_out)
    F1 = 2
    s1, s2 = slice(0, F1 * T), slice(F1 * T, F * T)
    part = {n: x[n][:, :, s1] for n in "qkvg"}
    _, S1, z1 = oracle.recurrent(oracle.FRAMECAUSAL, part["q"], part["k"], part["v"], part["g"],
                                 x["gamma"][:, :, :F1], S_in=x["S_in"], z_in=x["z_in"])
    b2 = oracle.backward(oracle.FRAMECAUSAL, x["q"][:, :, s2], x["k"][:, :, s2], x["v"][:, :, s2],
                         x["g"][:, :, s2], dO[:, :, s2], gamma=x["gamma"][:, :, F1:], S_in=S1,
                         z_in=z1, dS_out=dS_out, dz_out=dz_out)
    b1 = oracle.backward(oracle.FRAMECAUSAL, part["q"], part["k"], part["v"], part["g"],
                         dO[:, :, s1], gamma=x["gamma"][:, :, :F1], S_in=x["S_in"],
                         z_in=x["z_in"], dS_out=b2["dS_in"], dz_out=b2["dz_in"])
    for n in ("dq", "dk", "dv", "dg"):
        assert close(np.concatenate([b1[n], b2[n]], axis=2), full[n], 1e-11), n
    assert close(np.concatenate([b1["dgamma"], b2["dgamma"]], axis=2), full["dgamma"], 1e-11)
    assert close(b1["dS_in"], full["dS_in"], 1e-11) and close(b1["dz_in"], full["dz_in"], 1e-11)
