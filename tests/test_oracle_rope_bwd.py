"""Pins of the fp64 backward oracle with 3D rotary positions
(oracle.backward(..., rope=...)).

The rotary form (numerator on turned features, normaliser on unturned ones)
is pinned in its forward by test_oracle_rope.py; these pins tie its backward
to that forward and to the mathematics, never to the backward's own formulas:
- central finite differences of L = <dO, o> + <dS_out, S_out> + <dz_out, z_out>
  computed with the rotary forward oracle, for every input element, in both
  modes, with a nonzero frame offset and a carried state;
- positions all at the origin (one token per frame, one frame at offset 0)
  turn nothing, so the gradients are those without rotation;
- a stream cut into two blocks (the second continuing at frame_offset + F1,
  its dS_in fed back as the first block's dS_out) gives the one-shot
  gradients.
"""
from __future__ import annotations

import numpy as np

import oracle
from gla_testutil import close


def away_from_kinks(rng, shape, margin=0.2):
    x = rng.standard_normal(shape)
    return np.sign(x) * (margin + np.abs(x))


ROPE = dict(grid_h=1, grid_w=2, frame_offset=3, dim_t=2, dim_h=2, dim_w=2, theta=7.0)


def inputs(seed, B, H, F, T, d, causal=True):
    rng = np.random.default_rng(seed)
    x = {n: away_from_kinks(rng, (B, H, F * T, d)) for n in "qkv"}
    x["g"] = rng.standard_normal((B, H, F * T, d))
    if causal:
        x["gamma"] = rng.uniform(0.3, 0.95, (B, H, F))
        x["S_in"] = rng.standard_normal((B, H, d, d))
        x["z_in"] = rng.uniform(0.5, 2.0, (B, H, d))
    return x, rng


def loss(mode, x, dO, dS_out, dz_out, F, T, rope):
    if mode == oracle.BIDIR:
        o, _, _ = oracle.rope_recurrent(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], F=F, T=T,
                                        rope=rope)
        return float(np.sum(dO * o))
    o, S, z = oracle.rope_recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                    x["gamma"], x["S_in"], x["z_in"], rope=rope)
    return float(np.sum(dO * o) + np.sum(dS_out * S) + np.sum(dz_out * z))


def finite_differences(mode, x, dO, dS_out, dz_out, F, T, rope, h=1e-6):
    grads = {}
    for name, a in x.items():
        gd = np.empty_like(a)
        for idx in np.ndindex(a.shape):
            keep = a[idx]
            a[idx] = keep + h
            lp = loss(mode, x, dO, dS_out, dz_out, F, T, rope)
            a[idx] = keep - h
            lm = loss(mode, x, dO, dS_out, dz_out, F, T, rope)
            a[idx] = keep
            gd[idx] = (lp - lm) / (2 * h)
        grads[name] = gd
    return grads


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-12)


def test_framecausal_gradients_match_finite_differences():
    B, H, F, T, d = 1, 2, 3, 2, 6
    x, rng = inputs(41, B, H, F, T, d)
    dO = rng.standard_normal((B, H, F * T, d))
    dS_out = rng.standard_normal((B, H, d, d))
    dz_out = rng.standard_normal((B, H, d))
    got = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                          gamma=x["gamma"], S_in=x["S_in"], z_in=x["z_in"], dS_out=dS_out,
                          dz_out=dz_out, rope=ROPE)
    fd = finite_differences(oracle.FRAMECAUSAL, x, dO, dS_out, dz_out, F, T, ROPE)
    for a, b in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("gamma", "dgamma"),
                 ("S_in", "dS_in"), ("z_in", "dz_in")]:
        assert rel(got[b], fd[a]) < 1e-6, (a, rel(got[b], fd[a]))


def test_bidirectional_gradients_match_finite_differences():
    B, H, F, T, d = 1, 2, 3, 2, 6
    x, rng = inputs(42, B, H, F, T, d, causal=False)
    dO = rng.standard_normal((B, H, F * T, d))
    got = oracle.backward(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], dO, F=F, T=T, rope=ROPE)
    fd = finite_differences(oracle.BIDIR, x, dO, None, None, F, T, ROPE)
    for a in "qkvg":
        assert rel(got["d" + a], fd[a]) < 1e-6, (a, rel(got["d" + a], fd[a]))


def test_positions_at_the_origin_turn_nothing():
    B, H, F, T, d = 1, 2, 1, 1, 6
    x, rng = inputs(43, B, H, F, T, d)
    dO = rng.standard_normal((B, H, F * T, d))
    dS_out = rng.standard_normal((B, H, d, d))
    dz_out = rng.standard_normal((B, H, d))
    origin = dict(grid_h=1, grid_w=1, frame_offset=0, dim_t=2, dim_h=2, dim_w=2, theta=7.0)
    kw = dict(gamma=x["gamma"], S_in=x["S_in"], z_in=x["z_in"], dS_out=dS_out, dz_out=dz_out)
    args = (x["q"], x["k"], x["v"], x["g"], dO)
    got = oracle.backward(oracle.FRAMECAUSAL, *args, rope=origin, **kw)
    ref = oracle.backward(oracle.FRAMECAUSAL, *args, **kw)
    for n in ref:
        assert close(got[n], ref[n], 1e-13), n


def test_two_blocks_chain_at_their_absolute_positions():
    B, H, F, T, d = 1, 1, 5, 4, 8
    rope = dict(grid_h=2, grid_w=2, frame_offset=1, dim_t=2, dim_h=2, dim_w=4, theta=10.0)
    x, rng = inputs(44, B, H, F, T, d)
    dO = rng.standard_normal((B, H, F * T, d))
    dS_out = rng.standard_normal((B, H, d, d))
    dz_out = rng.standard_normal((B, H, d))
    full = oracle.backward(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], dO,
                           gamma=x["gamma"], S_in=x["S_in"], z_in=x["z_in"], dS_out=dS_out,
                           dz_out=dz_out, rope=rope)
    F1 = 2
    s1, s2 = slice(0, F1 * T), slice(F1 * T, F * T)
    rope2 = dict(rope, frame_offset=rope["frame_offset"] + F1)
    p1 = {n: x[n][:, :, s1] for n in "qkvg"}
    p2 = {n: x[n][:, :, s2] for n in "qkvg"}
    _, S1, z1 = oracle.rope_recurrent(oracle.FRAMECAUSAL, p1["q"], p1["k"], p1["v"], p1["g"],
                                      x["gamma"][:, :, :F1], x["S_in"], x["z_in"], rope=rope)
    b2 = oracle.backward(oracle.FRAMECAUSAL, p2["q"], p2["k"], p2["v"], p2["g"], dO[:, :, s2],
                         gamma=x["gamma"][:, :, F1:], S_in=S1, z_in=z1, dS_out=dS_out,
                         dz_out=dz_out, rope=rope2)
    b1 = oracle.backward(oracle.FRAMECAUSAL, p1["q"], p1["k"], p1["v"], p1["g"], dO[:, :, s1],
                         gamma=x["gamma"][:, :, :F1], S_in=x["S_in"], z_in=x["z_in"],
                         dS_out=b2["dS_in"], dz_out=b2["dz_in"], rope=rope)
    for n in ("dq", "dk", "dv", "dg", "dgamma"):
        assert close(np.concatenate([b1[n], b2[n]], axis=2), full[n], 1e-11), n
    assert close(b1["dS_in"], full["dS_in"], 1e-11) and close(b1["dz_in"], full["dz_in"], 1e-11)
