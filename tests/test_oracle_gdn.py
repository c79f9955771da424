"""Pins of the frame-wise Gated DeltaNet oracle (oracle.gdn).

Reading (the SANA-WM analysis page names the mixer and its 1/sqrt(D S) key
scaling, nothing more): one block delta-rule update per frame, every token of
the frame measuring its prediction error against the same decayed prior,
S = tokens per frame. The pins below tie the oracle to that definition by
properties it must have, not by retyping it.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from gla_testutil import close

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_worked_example_d1.json")


def rand(rng, B, H, F, T, d):
    q, k, v = (rng.standard_normal((B, H, F * T, d)) for _ in range(3))
    beta = rng.uniform(0.1, 1.0, (B, H, F * T))
    gamma = rng.uniform(0.5, 1.0, (B, H, F))
    return q, k, v, beta, gamma


def test_worked_example():
    g = json.load(open(GOLDEN))
    arr = {n: np.array(g[n], np.float64) for n in ("q", "k", "v", "beta", "gamma", "S_in")}
    o, S = oracle.gdn(arr["q"], arr["k"], arr["v"], arr["beta"], arr["gamma"], S_in=arr["S_in"],
                      key_scale=g["key_scale"])
    assert close(o, np.array(g["o"]), 1e-15)
    assert np.allclose(S, np.array(g["S_out"]), atol=1e-15)


def test_orthonormal_keys_are_recalled_exactly():
    """beta = 1 and a frame whose scaled keys are orthonormal: afterwards the
    state maps each key to its value, whatever the prior (delta rule), so a
    query equal to a key reads that key's value."""
    rng = np.random.default_rng(1)
    d, T, F = 6, 4, 3
    c = 0.37
    o_list, q_all, k_all, v_all = [], [], [], []
    for f in range(F):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        kt = Qm[:T]                       # orthonormal rows: the scaled keys
        k_all.append(kt / c)
        q_all.append(kt)
        v_all.append(rng.standard_normal((T, d)))
    k = np.concatenate(k_all)[None, None]
    q = np.concatenate(q_all)[None, None]
    v = np.concatenate(v_all)[None, None]
    gamma = rng.uniform(0.3, 1.0, (1, 1, F))
    S_in = rng.standard_normal((1, 1, d, d))
    o, _ = oracle.gdn(q, k, v, np.ones((1, 1, F * T)), gamma, S_in=S_in, key_scale=c)
    assert close(o, v, 1e-12)


def test_no_writes_only_decay():
    """beta = 0: S_f = (prod_{m <= f} gamma_m) S_in, so o_t = that times S_in^T q_t."""
    rng = np.random.default_rng(2)
    q, k, v, _, gamma = rand(rng, 1, 2, 4, 3, 5)
    S_in = rng.standard_normal((1, 2, 5, 5))
    o, S = oracle.gdn(q, k, v, np.zeros((1, 2, 12)), gamma, S_in=S_in)
    w = np.cumprod(gamma, axis=-1)  # [1, 2, F]
    want = np.einsum("bhnd,bhde->bhne", q, S_in) * np.repeat(w, 3, axis=-1)[..., None]
    assert close(o, want, 1e-13)
    assert close(S, S_in * w[..., -1:, None], 1e-13)


def test_rotation_of_the_key_space():
    """q -> q R, k -> k R (R orthogonal) with S_in -> R^T S_in: same outputs,
    S_out -> R^T S_out."""
    rng = np.random.default_rng(3)
    d = 5
    q, k, v, beta, gamma = rand(rng, 1, 2, 3, 4, d)
    S_in = rng.standard_normal((1, 2, d, d))
    R, _ = np.linalg.qr(rng.standard_normal((d, d)))
    o1, S1 = oracle.gdn(q, k, v, beta, gamma, S_in=S_in)
    o2, S2 = oracle.gdn(q @ R, k @ R, v, beta, gamma, S_in=R.T @ S_in)
    assert close(o2, o1, 1e-12)
    assert close(S2, R.T @ S1, 1e-12)


def test_linear_in_values_and_state():
    """Given q, k, beta, gamma the outputs are linear in (v, S_in) jointly."""
    rng = np.random.default_rng(4)
    q, k, v1, beta, gamma = rand(rng, 1, 1, 3, 5, 4)
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = (rng.standard_normal((1, 1, 4, 4)) for _ in range(2))
    a, Sa = oracle.gdn(q, k, v1, beta, gamma, S_in=s1)
    b, Sb = oracle.gdn(q, k, v2, beta, gamma, S_in=s2)
    c, Sc = oracle.gdn(q, k, 2 * v1 - 3 * v2, beta, gamma, S_in=2 * s1 - 3 * s2)
    assert close(c, 2 * a - 3 * b, 1e-12) and close(Sc, 2 * Sa - 3 * Sb, 1e-12)


def test_block_split_with_carry():
    rng = np.random.default_rng(5)
    q, k, v, beta, gamma = rand(rng, 1, 2, 5, 3, 4)
    T = 3
    o, S = oracle.gdn(q, k, v, beta, gamma, key_scale=0.2)
    s1, s2 = slice(0, 2 * T), slice(2 * T, 5 * T)
    o1, S1 = oracle.gdn(q[:, :, s1], k[:, :, s1], v[:, :, s1], beta[:, :, s1], gamma[:, :, :2],
                        key_scale=0.2)
    o2, S2 = oracle.gdn(q[:, :, s2], k[:, :, s2], v[:, :, s2], beta[:, :, s2], gamma[:, :, 2:],
                        S_in=S1, key_scale=0.2)
    assert close(np.concatenate([o1, o2], axis=2), o, 1e-12) and close(S2, S, 1e-12)


def test_key_scale_enters_through_the_keys_only():
    """Scaling the keys by a and key_scale by 1/a changes nothing; the default
    key_scale is 1/sqrt(d T)."""
    rng = np.random.default_rng(6)
    q, k, v, beta, gamma = rand(rng, 1, 2, 3, 4, 5)
    o1, S1 = oracle.gdn(q, k, v, beta, gamma, key_scale=0.3)
    o2, S2 = oracle.gdn(q, 2.5 * k, v, beta, gamma, key_scale=0.3 / 2.5)
    assert close(o1, o2, 1e-12) and close(S1, S2, 1e-12)
    o3, _ = oracle.gdn(q, k, v, beta, gamma)
    o4, _ = oracle.gdn(q, k, v, beta, gamma, key_scale=1 / np.sqrt(5 * 4))
    assert close(o3, o4, 1e-15)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_frame_order_matters_not_token_order(dtype):
    """Within a frame the update is a sum over tokens (all against the same
    prior): permuting a frame's tokens (with their beta) permutes its outputs
    and leaves the state unchanged."""
    rng = np.random.default_rng(7)
    q, k, v, beta, gamma = rand(rng, 1, 1, 2, 5, 3)
    perm = np.concatenate([np.arange(5), 5 + rng.permutation(5)])
    o, S = oracle.gdn(q.astype(dtype), k.astype(dtype), v.astype(dtype), beta, gamma)
    op, Sp = oracle.gdn(q[:, :, perm].astype(dtype), k[:, :, perm].astype(dtype),
                        v[:, :, perm].astype(dtype), beta[:, :, perm], gamma)
    assert close(op, o[:, :, perm], 1e-12) and close(Sp, S, 1e-12)
