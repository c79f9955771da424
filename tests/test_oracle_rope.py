"""Pins of the rotary (3D RoPE) variant of the fp64 oracle.

Reading taken for where the rotation sits (the SANA-Video ICLR 2026 oral talk
adds 3D RoPE to the linear attention but does not say where): RoFormer's rotary
linear attention -- rotated phi(q), phi(k) in the numerator, unrotated in the
normaliser. The pins below fix that reading, the position of each token, the
section/frequency schedule and the direction of rotation.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gla_testutil import close


def rand(rng, B, H, F, T, d):
    q, k, v, g = (rng.standard_normal((B, H, F * T, d)) for _ in range(4))
    gamma = expit(rng.normal(1.0, 1.0, size=(B, H, F)))
    return q, k, v, g, gamma


@pytest.mark.parametrize("seed", range(4))
def test_recurrent_equals_quadratic(seed):
    rng = np.random.default_rng(300 + seed)
    B, H, F, gh, gw = 1, 2, 3, 2, 3
    d = 12
    q, k, v, g, gamma = rand(rng, B, H, F, gh * gw, d)
    rope = dict(grid_h=gh, grid_w=gw, frame_offset=int(rng.integers(0, 9)), dim_t=4, dim_h=4,
                dim_w=4, theta=float(rng.uniform(2.0, 50.0)))
    S_in = rng.standard_normal((B, H, d, d))
    z_in = np.abs(rng.standard_normal((B, H, d)))
    for mode in (oracle.BIDIR, oracle.FRAMECAUSAL):
        kw = dict(F=F, T=gh * gw) if mode == oracle.BIDIR else dict(S_in=S_in, z_in=z_in)
        a = oracle.rope_recurrent(mode, q, k, v, g, gamma, rope=rope, **kw)[0]
        b = oracle.rope_quadratic(mode, q, k, v, g, gamma, rope=rope, **kw)
        assert close(a, b, 1e-12)


def test_zero_angles_reduce_to_unrotated():
    """Every pair in the temporal section and a single frame at t = 0: no
    rotation at all, so the rotary oracle equals the plain one."""
    rng = np.random.default_rng(1)
    q, k, v, g, gamma = rand(rng, 1, 2, 1, 6, 8)
    rope = dict(grid_h=2, grid_w=3, frame_offset=0, dim_t=8, dim_h=0, dim_w=0, theta=10.0)
    for mode in (oracle.BIDIR, oracle.FRAMECAUSAL):
        a = oracle.rope_recurrent(mode, q, k, v, g, gamma, rope=rope,
                                  **(dict(F=1, T=6) if mode == oracle.BIDIR else {}))
        b = oracle.recurrent(mode, q, k, v, g, gamma)
        for x, y in zip(a, b):
            assert close(x, y, 1e-13)


def test_shift_invariance_of_frame_offset():
    """Rotations enter only through position differences: shifting every
    frame's temporal position leaves the outputs unchanged."""
    rng = np.random.default_rng(2)
    q, k, v, g, gamma = rand(rng, 1, 2, 4, 6, 12)
    base = dict(grid_h=2, grid_w=3, dim_t=4, dim_h=4, dim_w=4, theta=7.0)
    a = oracle.rope_recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma,
                              rope=dict(base, frame_offset=0))[0]
    b = oracle.rope_recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma,
                              rope=dict(base, frame_offset=37))[0]
    assert close(a, b, 1e-11)
    # ... whereas moving the spatial grid does change them (the rotation acts)
    c = oracle.rope_recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma,
                              rope=dict(base, frame_offset=0, grid_h=3, grid_w=2))[0]
    assert not close(a, c, 1e-6)


def test_single_token_closed_form():
    """One token at any position: rotations are orthogonal, so the numerator
    is phi(q).phi(k) v and o = sigmoid(g) v a / (a + eps)."""
    rng = np.random.default_rng(3)
    d = 6
    q, k, v, g = (rng.standard_normal((1, 1, 1, d)) for _ in range(4))
    a = float(np.maximum(q, 0).ravel() @ np.maximum(k, 0).ravel())
    rope = dict(grid_h=1, grid_w=1, frame_offset=5, dim_t=2, dim_h=2, dim_w=2, theta=3.0)
    o = oracle.rope_recurrent(oracle.FRAMECAUSAL, q, k, v, g, np.ones((1, 1, 1)), rope=rope,
                              eps=0.25)[0]
    assert close(o, expit(g) * v * a / (a + 0.25), 1e-13)


@pytest.mark.parametrize("section", ["t", "h", "w"])
def test_frequency_schedule_and_direction(section):
    """Bidirectional, two key tokens, and a query whose only nonzero feature is
    the first of pair p; key s has only the first (or only the second) feature
    of pair p. With eps = 0 and v one-hot the output ratio is
    cos(dpos * f_p) (or sin(dpos * f_p)), f_p = theta^(-j/m) for the pair's
    index j within its section of m pairs, dpos the query's position minus the
    key's along that section's axis."""
    gh, gw, F, theta = 3, 4, 3, 5.0
    T = gh * gw
    dims = dict(dim_t=4, dim_h=6, dim_w=6)
    d = sum(dims.values())
    Pt, Ph = dims["dim_t"] // 2, dims["dim_h"] // 2
    pairs = {"t": range(0, Pt), "h": range(Pt, Pt + Ph), "w": range(Pt + Ph, d // 2)}[section]
    first = {"t": 0, "h": Pt, "w": Pt + Ph}[section]
    m = len(pairs)
    # query: frame 1, (y, x) = (2, 3); key: frame 0, (y, x) = (0, 0): the three
    # position differences (1, 2, 3) are distinct, so a swapped axis shows
    tq, tk = 1 * T + 2 * gw + 3, 0
    dpos = {"t": 1, "h": 2, "w": 3}[section]
    for p in pairs:
        for second in (False, True):
            N = F * T
            q = -np.ones((1, 1, N, d))
            k = -np.ones((1, 1, N, d))
            v = np.zeros((1, 1, N, d))
            g = np.full((1, 1, N, d), 50.0)  # sigmoid(50) == 1 in fp64
            q[0, 0, tq, :] = 0.0
            q[0, 0, tq, 2 * p] = 1.5
            k[0, 0, tk, :] = 0.0
            k[0, 0, tk, 2 * p + (1 if second else 0)] = 2.0
            v[0, 0, tk, 0] = 1.0
            # keep the normaliser away from zero: a second key, unrotated weight
            k[0, 0, tk + 1, :] = 0.0
            k[0, 0, tk + 1, 2 * p] = 1.0
            rope = dict(grid_h=gh, grid_w=gw, frame_offset=0, theta=theta, **dims)
            o = oracle.rope_recurrent(oracle.BIDIR, q, k, v, g, F=F, T=T, rope=rope,
                                      eps=0.0)[0]
            den = 1.5 * 0.0 + 1.5 * 1.0  # unrotated: only the second key's pair-p feature meets q
            if not second:
                den = 1.5 * 2.0 + 1.5 * 1.0
            f_p = theta ** (-(p - first) / m)
            want = 1.5 * 2.0 * (math.sin(dpos * f_p) if second else math.cos(dpos * f_p)) / den
            assert abs(o[0, 0, tq, 0] - want) < 1e-12, (section, p, second)


def test_worked_quarter_turn():
    """Hand-computed: d = 4 (two temporal pairs), theta = (pi/2)^-2 so that pair 1
    turns by a quarter per frame and pair 0 by one radian per frame. Query at
    frame 1, key at frame 0, q = k = (0, 0, 1, 0), v = e_0, eps = 0:
    num = (R_1 q) . (R_0 k) = cos(pi/2) = 0, so o = 0; with k = (0, 0, 0, 1)
    instead, (R_1 q).(R_0 k) = sin(pi/2) = 1 and den = q . k_unrotated."""
    theta = (math.pi / 2) ** -2
    rope = dict(grid_h=1, grid_w=1, frame_offset=0, dim_t=4, dim_h=0, dim_w=0, theta=theta)
    q = np.array([-1, -1, -1, -1, 0, 0, 1, 0], float).reshape(1, 1, 2, 4)
    k = np.array([0, 0, 1, 0, -1, -1, -1, -1], float).reshape(1, 1, 2, 4)
    v = np.array([1, 0, 0, 0, 0, 0, 0, 0], float).reshape(1, 1, 2, 4)
    g = np.full((1, 1, 2, 4), 60.0)
    o = oracle.rope_recurrent(oracle.BIDIR, q, k, v, g, F=2, T=1, rope=rope, eps=1e-3)[0]
    assert abs(o[0, 0, 1, 0]) < 1e-12  # cos(pi/2) numerator
    # second feature of the pair: sin(pi/2) = 1; normaliser phi(q).phi(k) = 0 + eps
    k2 = np.array([0, 0, 0, 1, -1, -1, -1, -1], float).reshape(1, 1, 2, 4)
    o2 = oracle.rope_recurrent(oracle.BIDIR, q, k2, v, g, F=2, T=1, rope=rope, eps=0.5)[0]
    assert abs(o2[0, 0, 1, 0] - 1.0 / 0.5) < 1e-12


def test_block_split_with_carry_needs_absolute_frame_offset():
    """Streaming with rotation: the carried state holds keys rotated at their
    absolute positions, so the second block must pass its frame offset; then
    block split == one shot (and with a wrong offset it is not)."""
    rng = np.random.default_rng(4)
    gh, gw, F, d = 2, 2, 4, 8
    T = gh * gw
    q, k, v, g, gamma = rand(rng, 1, 2, F, T, d)
    base = dict(grid_h=gh, grid_w=gw, dim_t=4, dim_h=2, dim_w=2, theta=3.0)
    o, S, z = oracle.rope_recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma,
                                    rope=dict(base, frame_offset=0))
    sl1, sl2 = slice(0, 2 * T), slice(2 * T, 4 * T)
    o1, S1, z1 = oracle.rope_recurrent(oracle.FRAMECAUSAL, q[:, :, sl1], k[:, :, sl1],
                                       v[:, :, sl1], g[:, :, sl1], gamma[:, :, :2],
                                       rope=dict(base, frame_offset=0))
    o2, S2, z2 = oracle.rope_recurrent(oracle.FRAMECAUSAL, q[:, :, sl2], k[:, :, sl2],
                                       v[:, :, sl2], g[:, :, sl2], gamma[:, :, 2:], S_in=S1,
                                       z_in=z1, rope=dict(base, frame_offset=2))
    assert close(np.concatenate([o1, o2], axis=2), o, 1e-12)
    assert close(S2, S, 1e-12) and close(z2, z, 1e-12)
    o2w = oracle.rope_recurrent(oracle.FRAMECAUSAL, q[:, :, sl2], k[:, :, sl2], v[:, :, sl2],
                                g[:, :, sl2], gamma[:, :, 2:], S_in=S1, z_in=z1,
                                rope=dict(base, frame_offset=0))[0]
    assert not close(o2w, o[:, :, sl2], 1e-6)
