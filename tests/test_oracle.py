"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the part of the method it pins and the mistake it would catch.
Sources: the gated linear attention token mixer of "SANA-Video 2.0" (section
"Hybrid Linear-Softmax Attention"), the fixed D x D state with an additive
per-block update (SANA-Video ICLR 2026 oral talk, block KV cache passage) and
frame-wise decay gates ("SANA-WM" analysis page, method components).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gla_testutil import close
from gated_linear_attention_fwd_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
FORMS = ("recurrent", "quadratic", "chunked")


def run(form, mode, *args, **kw):
    fn = getattr(oracle, form)
    return fn(mode, *args, **kw)


def rand_f64(rng, B, H, F, T, d, gmu=1.0, gsd=1.0):
    N = F * T
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    gamma = expit(rng.normal(gmu, gsd, size=(B, H, F)))
    return q, k, v, g, gamma


# ---------------------------------------------------------------- worked example

def _frac(x):
    return float(Fraction(x))


def _golden():
    with open(os.path.join(HERE, "golden", "worked_example_d2.json")) as f:
        ex = json.load(f)
    arr = lambda a: np.asarray(a, np.float64).reshape(1, 1, -1, ex["d"])
    gv = {"0": 0.0, "ln3": np.log(3.0), "-ln3": -np.log(3.0)}
    g = np.asarray([[gv[x] for x in row] for row in ex["g"]]).reshape(1, 1, -1, ex["d"])
    return ex, arr(ex["q"]), arr(ex["k"]), arr(ex["v"]), g, np.asarray(ex["gamma"]).reshape(1, 1, -1)


@pytest.mark.parametrize("form", FORMS)
def test_worked_example(form):
    """Hand-derived fractions (tests/golden/worked_example_d2.json): catches a
    transposed state, a missing ReLU, a gate with the wrong sign, decay applied
    after the frame's update, an exclusive (previous-frame) readout."""
    ex, q, k, v, g, gamma = _golden()
    d = ex["d"]
    fr = lambda a: np.vectorize(_frac)(np.asarray(a, dtype=object)).astype(np.float64)
    o, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma, eps=0.0)
    assert close(o.reshape(-1, d), fr(ex["framecausal"]["o"]), 1e-14)
    assert close(S.reshape(d, d), fr(ex["framecausal"]["S_out"]), 1e-14)
    assert close(z.reshape(d), fr(ex["framecausal"]["z_out"]), 1e-14)
    c = ex["framecausal_carry"]
    o, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma, S_in=np.asarray(c["S_in"], float),
                  z_in=np.asarray(c["z_in"], float), eps=0.0)
    assert close(o.reshape(-1, d), fr(c["o"]), 1e-14)
    assert close(S.reshape(d, d), fr(c["S_out"]), 1e-14)
    assert close(z.reshape(d), fr(c["z_out"]), 1e-14)
    o, S, z = run(form, oracle.BIDIR, q, k, v, g, eps=0.0)
    assert close(o.reshape(-1, d), fr(ex["bidir"]["o"]), 1e-14)
    assert close(S.reshape(d, d), fr(ex["bidir"]["S_out"]), 1e-14)
    assert close(z.reshape(d), fr(ex["bidir"]["z_out"]), 1e-14)


# ---------------------------------------------------------------- three forms agree

@pytest.mark.parametrize("seed", range(6))
def test_forms_agree_random_shapes(seed):
    """Recurrent == quadratic == chunked (C=7 and C=T) on random tiny shapes,
    with and without a carried state, both modes."""
    rng = np.random.default_rng(100 + seed)
    B, H = rng.integers(1, 3, 2)
    d = int(rng.choice([2, 3, 5, 8, 16]))
    F, T = int(rng.integers(1, 5)), int(rng.integers(1, 10))
    q, k, v, g, gamma = rand_f64(rng, B, H, F, T, d)
    S_in = rng.standard_normal((B, H, d, d))
    z_in = np.abs(rng.standard_normal((B, H, d)))
    for mode in (oracle.BIDIR, oracle.FRAMECAUSAL):
        for carry in (False, True):
            kw = dict(S_in=S_in, z_in=z_in) if carry else {}
            r = oracle.recurrent(mode, q, k, v, g, gamma, **kw)
            for other in (oracle.quadratic(mode, q, k, v, g, gamma, **kw),
                          oracle.chunked(mode, q, k, v, g, gamma, C=7, **kw),
                          oracle.chunked(mode, q, k, v, g, gamma, C=T, **kw)):
                for a, b in zip(other, r):
                    assert close(a, b, 1e-11)


@pytest.mark.parametrize("mode", [oracle.BIDIR, oracle.FRAMECAUSAL])
def test_forms_agree_tiny_workload(mode):
    """The tiny fp32 workload (B=1, H=2, d=16, 4 frames x 16 tokens) in all three forms."""
    w = synth.WORKLOADS[1]
    x = synth.workload_inputs(w)
    args = (x["q"], x["k"], x["v"], x["g"], x["gamma"])
    r = oracle.recurrent(mode, *args)
    for other in (oracle.quadratic(mode, *args), oracle.chunked(mode, *args, C=7),
                  oracle.chunked(mode, *args, C=w.T)):
        for a, b in zip(other, r):
            assert close(a, b, 1e-12)


def test_bf16_inputs_upcast_exactly():
    """bf16 bit patterns give the same result as their exact float64 values."""
    rng = np.random.default_rng(7)
    x = synth.random_inputs(1, 2, 3, 5, 8, "bf16", seed=7)
    as64 = {n: oracle.bf16_to_f64(x[n]) for n in "qkvg"}
    a = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["gamma"])
    b = oracle.recurrent(oracle.FRAMECAUSAL, as64["q"], as64["k"], as64["v"], as64["g"],
                         x["gamma"])
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
    del rng


# ---------------------------------------------------------------- closed forms (a1, a5)

@pytest.mark.parametrize("form", FORMS)
def test_single_token_closed_form(form):
    """N = 1: o = sigmoid(g) v a / (a + eps) with a = phi(q).phi(k). Catches a
    transposed readout (phi(k)(phi(q).v)), eps in the wrong place, missing ReLU."""
    rng = np.random.default_rng(3)
    d = 6
    q, k, v, g = (rng.standard_normal((1, 1, 1, d)) for _ in range(4))
    eps = 0.25
    a = float(np.maximum(q, 0).ravel() @ np.maximum(k, 0).ravel())
    want = expit(g) * v * a / (a + eps)
    o, _, _ = run(form, oracle.BIDIR, q, k, v, g, eps=eps)
    assert close(o, want, 1e-13)


@pytest.mark.parametrize("mode", [oracle.BIDIR, oracle.FRAMECAUSAL])
@pytest.mark.parametrize("form", FORMS)
def test_constant_values_weighted_average(mode, form):
    """v_t = c for every token: o = sigmoid(g) c den/(den+eps); with eps = 0,
    o = sigmoid(g) c exactly. Catches a normaliser that is not decayed like S."""
    rng = np.random.default_rng(4)
    B, H, F, T, d = 1, 2, 3, 5, 4
    q, k, _, g, gamma = rand_f64(rng, B, H, F, T, d)
    q = np.abs(q)  # every query sees a positive normaliser
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, q.shape).copy()
    o, _, _ = run(form, mode, q, k, v, g, gamma, eps=0.0)
    assert close(o, expit(g) * c, 1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_gate_is_logistic_sigmoid(form):
    """v = 1, eps = 0: o = sigmoid(g), compared with scipy's expit."""
    rng = np.random.default_rng(5)
    q, k, _, g, gamma = rand_f64(rng, 1, 1, 2, 4, 3)
    q = np.abs(q)
    g = 4.0 * g
    o, _, _ = run(form, oracle.FRAMECAUSAL, q, k, np.ones_like(q), g, gamma, eps=0.0)
    assert close(o, expit(g), 1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_nonpositive_queries_give_zero(form):
    """phi(q) = 0 gives o = 0 exactly (0 / (0 + eps)). Catches a missing ReLU on q."""
    rng = np.random.default_rng(6)
    q, k, v, g, gamma = rand_f64(rng, 1, 2, 2, 3, 4)
    o, _, _ = run(form, oracle.FRAMECAUSAL, -np.abs(q), k, v, g, gamma)
    assert np.all(o == 0.0)


@pytest.mark.parametrize("form", FORMS)
def test_nonpositive_keys_give_zero(form):
    """phi(k) = 0 leaves S = 0 and z = 0, hence o = 0. Catches a missing ReLU on k."""
    rng = np.random.default_rng(8)
    q, k, v, g, gamma = rand_f64(rng, 1, 2, 2, 3, 4)
    o, S, z = run(form, oracle.FRAMECAUSAL, q, -np.abs(k), v, g, gamma)
    assert np.all(o == 0.0) and np.all(S == 0.0) and np.all(z == 0.0)


# ---------------------------------------------------------------- scan (a3)

@pytest.mark.parametrize("form", FORMS)
def test_scan_geometric_closed_form(form):
    """Identical frames and constant gamma: S_f = U (1 - gamma^(f+1)) / (1 - gamma).
    U is the frame's phi(K)^T V from a numpy matmul. Catches decay applied after
    the update (which would give gamma (1 - gamma^(f+1)) / (1 - gamma))."""
    rng = np.random.default_rng(9)
    F, T, d, gm = 5, 4, 3, 0.7
    kf, vf = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    k = np.tile(kf, (F, 1)).reshape(1, 1, F * T, d)
    v = np.tile(vf, (F, 1)).reshape(1, 1, F * T, d)
    q = g = np.zeros_like(k)
    U = np.maximum(kf, 0).T @ vf
    u = np.maximum(kf, 0).sum(0)
    _, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, np.full((1, 1, F), gm))
    geo = (1 - gm ** F) / (1 - gm)
    assert close(S.reshape(d, d), U * geo, 1e-13)
    assert close(z.reshape(d), u * geo, 1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_decay_indexing(form):
    """Only frame j carries keys: S_out = (prod_{m=j+1}^{F-1} gamma_m) U_j, with a
    distinct gamma per frame. Catches an off-by-one in the decay index."""
    rng = np.random.default_rng(10)
    F, T, d = 5, 3, 4
    gamma = np.array([0.9, 0.8, 0.6, 0.5, 0.3]).reshape(1, 1, F)
    for j in range(F):
        k = -np.abs(rng.standard_normal((1, 1, F * T, d)))
        v = np.zeros((1, 1, F * T, d))
        kj, vj = rng.standard_normal((T, d)), rng.standard_normal((T, d))
        k[0, 0, j * T:(j + 1) * T] = kj
        v[0, 0, j * T:(j + 1) * T] = vj
        _, S, z = run(form, oracle.FRAMECAUSAL, np.zeros_like(k), k, v, np.zeros_like(k), gamma)
        w = np.prod(gamma.ravel()[j + 1:])
        assert close(S.reshape(d, d), w * (np.maximum(kj, 0).T @ vj), 1e-13)
        assert close(z.reshape(d), w * np.maximum(kj, 0).sum(0), 1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_carry_single_frame(form):
    """F = 1 with a carried state: S_out = gamma_0 S_in + U_0, z likewise."""
    rng = np.random.default_rng(11)
    T, d = 6, 5
    q, k, v, g, _ = rand_f64(rng, 1, 1, 1, T, d)
    S_in, z_in = rng.standard_normal((d, d)), np.abs(rng.standard_normal(d))
    gm = 0.35
    _, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, np.full((1, 1, 1), gm),
                  S_in=S_in, z_in=z_in)
    U = np.maximum(k[0, 0], 0).T @ v[0, 0]
    assert close(S.reshape(d, d), gm * S_in + U, 1e-13)
    assert close(z.reshape(d), gm * z_in + np.maximum(k[0, 0], 0).sum(0), 1e-13)


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("form", FORMS)
def test_gamma_zero_each_frame_is_bidirectional(form):
    """gamma = 0 resets the state: every frame equals bidirectional attention over
    that frame alone."""
    rng = np.random.default_rng(12)
    B, H, F, T, d = 1, 2, 3, 4, 5
    q, k, v, g, _ = rand_f64(rng, B, H, F, T, d)
    o, _, _ = run(form, oracle.FRAMECAUSAL, q, k, v, g, np.zeros((B, H, F)))
    for f in range(F):
        sl = slice(f * T, (f + 1) * T)
        ob, _, _ = run(form, oracle.BIDIR, q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, sl])
        assert close(o[:, :, sl], ob, 1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_single_frame_equals_bidirectional(form):
    rng = np.random.default_rng(13)
    q, k, v, g, gamma = rand_f64(rng, 2, 1, 1, 9, 4)
    a = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma)
    b = run(form, oracle.BIDIR, q, k, v, g)
    for x, y in zip(a, b):
        assert close(x, y, 1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_gamma_one_last_frame_equals_bidirectional(form):
    """gamma = 1: the last frame's outputs equal the bidirectional outputs. Catches
    a readout that excludes the token's own frame."""
    rng = np.random.default_rng(14)
    B, H, F, T, d = 1, 2, 4, 3, 4
    q, k, v, g, _ = rand_f64(rng, B, H, F, T, d)
    o, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, np.ones((B, H, F)))
    ob, Sb, zb = run(form, oracle.BIDIR, q, k, v, g)
    assert close(o[:, :, -T:], ob[:, :, -T:], 1e-12)
    assert close(S, Sb, 1e-12) and close(z, zb, 1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_permutation_within_frame(form):
    """Permuting the tokens of a frame permutes their outputs; permuting only (k, v)
    inside a frame leaves every output unchanged."""
    rng = np.random.default_rng(15)
    B, H, F, T, d = 1, 1, 3, 6, 4
    q, k, v, g, gamma = rand_f64(rng, B, H, F, T, d)
    o, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma)
    perm = np.arange(F * T)
    perm[T:2 * T] = T + rng.permutation(T)
    o2, S2, z2 = run(form, oracle.FRAMECAUSAL, q[:, :, perm], k[:, :, perm], v[:, :, perm],
                     g[:, :, perm], gamma)
    assert close(o2, o[:, :, perm], 1e-12) and close(S2, S, 1e-12) and close(z2, z, 1e-12)
    o3, _, _ = run(form, oracle.FRAMECAUSAL, q, k[:, :, perm], v[:, :, perm], g, gamma)
    assert close(o3, o, 1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_causality_across_frames(form):
    """Changing frames after f leaves the outputs of frames <= f bit-identical."""
    rng = np.random.default_rng(16)
    B, H, F, T, d = 1, 2, 4, 3, 4
    q, k, v, g, gamma = rand_f64(rng, B, H, F, T, d)
    o, _, _ = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma)
    cut = 2 * T
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:, :, cut:] = rng.standard_normal(k2[:, :, cut:].shape)
    v2[:, :, cut:] += 3.0
    q2[:, :, cut:] *= -1
    o2, _, _ = run(form, oracle.FRAMECAUSAL, q2, k2, v2, g, gamma)
    assert np.array_equal(o2[:, :, :cut], o[:, :, :cut])


@pytest.mark.parametrize("form", FORMS)
def test_block_split_equals_one_shot(form):
    """Carrying (S, z) across blocks of frames gives the one-shot result: the
    block KV cache of the talk, with decay."""
    rng = np.random.default_rng(17)
    B, H, F, T, d = 1, 2, 7, 3, 4
    q, k, v, g, gamma = rand_f64(rng, B, H, F, T, d)
    o, S, z = run(form, oracle.FRAMECAUSAL, q, k, v, g, gamma)
    Sc = zc = None
    outs = []
    for f0, f1 in ((0, 2), (2, 3), (3, 7)):
        sl = slice(f0 * T, f1 * T)
        ob, Sc, zc = run(form, oracle.FRAMECAUSAL, q[:, :, sl], k[:, :, sl], v[:, :, sl],
                         g[:, :, sl], gamma[:, :, f0:f1], S_in=Sc, z_in=zc)
        outs.append(ob)
    assert close(np.concatenate(outs, axis=2), o, 1e-12)
    assert close(Sc, S, 1e-12) and close(zc, z, 1e-12)
    # state-only commit gives the same state
    _, Ss, zs = run(form, oracle.FRAMECAUSAL, None, k, v, None, gamma, outputs=False)
    assert close(Ss, S, 1e-12) and close(zs, z, 1e-12)


@pytest.mark.parametrize("mode", [oracle.BIDIR, oracle.FRAMECAUSAL])
def test_linearity_in_values(mode):
    """o(a V1 + b V2) = a o(V1) + b o(V2) at fixed q, k, g."""
    rng = np.random.default_rng(18)
    q, k, v1, g, gamma = rand_f64(rng, 1, 2, 3, 4, 5)
    v2 = rng.standard_normal(v1.shape)
    a, b = 1.7, -0.4
    o1 = oracle.recurrent(mode, q, k, v1, g, gamma)[0]
    o2 = oracle.recurrent(mode, q, k, v2, g, gamma)[0]
    o12 = oracle.recurrent(mode, q, k, a * v1 + b * v2, g, gamma)[0]
    assert close(o12, a * o1 + b * o2, 1e-12)


@pytest.mark.parametrize("mode", [oracle.BIDIR, oracle.FRAMECAUSAL])
def test_query_scale_invariance(mode):
    """At eps = 0 the readout is a ratio: o(c q) = o(q) for c > 0."""
    rng = np.random.default_rng(19)
    q, k, v, g, gamma = rand_f64(rng, 1, 2, 3, 4, 5)
    q = np.abs(q)
    a = oracle.recurrent(mode, q, k, v, g, gamma, eps=0.0)[0]
    b = oracle.recurrent(mode, 8.0 * q, k, v, g, gamma, eps=0.0)[0]
    assert close(a, b, 1e-13)


def test_zero_decay_frame_ignores_carry():
    """gamma_0 = 0 discards a carried state entirely."""
    rng = np.random.default_rng(20)
    q, k, v, g, gamma = rand_f64(rng, 1, 1, 2, 3, 4)
    gamma[..., 0] = 0.0
    a = oracle.recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma)
    b = oracle.recurrent(oracle.FRAMECAUSAL, q, k, v, g, gamma,
                         S_in=rng.standard_normal((4, 4)), z_in=np.ones(4))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_threads_do_not_change_results():
    """The OpenMP split over column blocks changes no arithmetic."""
    x = synth.random_inputs(1, 3, 3, 7, 20, "bf16", seed=21)
    a = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["gamma"],
                         nthreads=1)
    b = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["gamma"],
                         nthreads=4)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
