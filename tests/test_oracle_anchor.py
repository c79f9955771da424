"""Pins of the gated softmax anchor oracle (oracle.softmax_anchor).

Reading (the pages name the layer -- a gated-softmax anchor in one layer of
four, with attention-sink tokens and a local temporal window for deployment --
but print no formula): o_t = sigma(g_t) * sum over the visible keys of
softmax(scale q.k) v; visible = every key (full mode), or whole key frames i
<= f with i < n_sink or i > f - window (frame-causal). The pins tie the oracle
to that reading through a hand-derived example, a library routine and
properties, never by retyping it.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
from gla_testutil import close

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "anchor_worked_example_d1.json")


def rand(rng, B, H, Fq, F, T, d):
    q, g = (rng.standard_normal((B, H, Fq * T, d)) for _ in range(2))
    k, v = (rng.standard_normal((B, H, F * T, d)) for _ in range(2))
    return q, k, v, g


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def test_worked_example():
    e = json.load(open(GOLDEN))
    arr = {n: np.array(e[n], np.float64).reshape(1, 1, -1, 1) for n in "qkvg"}
    kw = dict(T=e["T"], n_sink=e["n_sink"], window=e["window"], scale=e["scale"])
    o = oracle.softmax_anchor(arr["q"], arr["k"], arr["v"], arr["g"], causal=True, **kw)
    assert close(o.ravel(), np.array(e["o_causal"]), 1e-14)
    o = oracle.softmax_anchor(arr["q"], arr["k"], arr["v"], arr["g"], causal=False, **kw)
    assert close(o.ravel(), np.array(e["o_full"]), 1e-14)
    # the last two frames as a streaming call over all four key frames
    o = oracle.softmax_anchor(arr["q"][:, :, 2:], arr["k"], arr["v"], arr["g"][:, :, 2:],
                              causal=True, **kw)
    assert close(o.ravel(), np.array(e["o_causal"][2:]), 1e-14)


@pytest.mark.parametrize("scale", [None, 0.3])
def test_full_mode_is_scaled_dot_product_attention(scale):
    """Full mode against torch's scaled_dot_product_attention (fp64, CPU) and
    the sigmoid gate."""
    rng = np.random.default_rng(1)
    q, k, v, g = rand(rng, 2, 3, 5, 5, 4, 8)
    o = oracle.softmax_anchor(q, k, v, g, T=4, causal=False, scale=scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    assert close(o, sig(g) * ref, 1e-12)


@pytest.mark.parametrize("n_sink,window", [(0, 0), (1, 2), (2, 3), (0, 1), (3, 1), (9, 2)])
def test_causal_equals_full_attention_over_the_kept_frames(n_sink, window):
    """Frame-causal output of query frame f equals full-mode attention over a
    key sequence built by keeping only the sink frames and the window frames
    (listed here as frame ranges, not tested one by one)."""
    rng = np.random.default_rng(2)
    F, T, d = 7, 3, 5
    q, k, v, g = rand(rng, 1, 2, F, F, T, d)
    o = oracle.softmax_anchor(q, k, v, g, T=T, causal=True, n_sink=n_sink, window=window)
    for f in range(F):
        first_window = 0 if window <= 0 else max(0, f - window + 1)
        kept = sorted(set(range(min(n_sink, f + 1))) | set(range(first_window, f + 1)))
        rows = np.concatenate([np.arange(i * T, (i + 1) * T) for i in kept])
        sl = slice(f * T, (f + 1) * T)
        want = oracle.softmax_anchor(q[:, :, sl], k[:, :, rows], v[:, :, rows], g[:, :, sl], T=T,
                                     causal=False)
        assert close(o[:, :, sl], want, 1e-13), (f, kept)


def test_streaming_rows_equal_the_full_call():
    rng = np.random.default_rng(3)
    F, T, d = 6, 4, 3
    q, k, v, g = rand(rng, 1, 2, F, F, T, d)
    full = oracle.softmax_anchor(q, k, v, g, T=T, causal=True, n_sink=1, window=2)
    for Fq in (1, 2, 5):
        sl = slice((F - Fq) * T, F * T)
        part = oracle.softmax_anchor(q[:, :, sl], k, v, g[:, :, sl], T=T, causal=True, n_sink=1,
                                     window=2)
        assert close(part, full[:, :, sl], 1e-14)


def test_unlimited_window_last_frame_sees_everything():
    rng = np.random.default_rng(4)
    F, T, d = 5, 3, 4
    q, k, v, g = rand(rng, 1, 1, F, F, T, d)
    causal = oracle.softmax_anchor(q, k, v, g, T=T, causal=True)
    full = oracle.softmax_anchor(q, k, v, g, T=T, causal=False)
    last = slice((F - 1) * T, F * T)
    assert close(causal[:, :, last], full[:, :, last], 1e-13)
    # and the first frame sees only itself
    first = slice(0, T)
    own = oracle.softmax_anchor(q[:, :, first], k[:, :, first], v[:, :, first], g[:, :, first],
                                T=T, causal=False)
    assert close(causal[:, :, first], own, 1e-13)


def test_constant_values_pass_through():
    rng = np.random.default_rng(5)
    F, T, d = 4, 5, 3
    q, k, _, g = rand(rng, 1, 2, F, F, T, d)
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, k.shape).copy()
    o = oracle.softmax_anchor(q, k, v, g, T=T, causal=True, n_sink=1, window=2)
    assert close(o, sig(g) * c, 1e-13)


def test_zero_queries_average_the_visible_values():
    """q = 0: every visible key weighs the same. Frame 4 of 6 with one sink
    frame and a window of 2 sees frames {0, 3, 4}."""
    rng = np.random.default_rng(6)
    F, T, d = 6, 2, 3
    _, k, v, g = rand(rng, 1, 1, F, F, T, d)
    q = np.zeros((1, 1, F * T, d))
    o = oracle.softmax_anchor(q, k, v, g, T=T, causal=True, n_sink=1, window=2)
    seen = np.concatenate([v[0, 0, 0:2], v[0, 0, 6:8], v[0, 0, 8:10]])
    assert close(o[0, 0, 8:10], sig(g[0, 0, 8:10]) * seen.mean(axis=0), 1e-14)


def test_common_key_offset_changes_nothing():
    """Adding the same vector u to every key shifts each query's scores by
    q.u, which softmax ignores."""
    rng = np.random.default_rng(7)
    q, k, v, g = rand(rng, 1, 2, 3, 4, 3, 4)
    u = 3.0 * rng.standard_normal(4)
    a = oracle.softmax_anchor(q, k, v, g, T=3, causal=True, n_sink=1, window=2)
    b = oracle.softmax_anchor(q, k + u, v, g, T=3, causal=True, n_sink=1, window=2)
    assert close(a, b, 1e-12)


def test_key_order_within_a_frame_does_not_matter():
    rng = np.random.default_rng(8)
    F, T = 4, 5
    q, k, v, g = rand(rng, 1, 1, F, F, T, 3)
    perm = np.concatenate([f * T + rng.permutation(T) for f in range(F)])
    a = oracle.softmax_anchor(q, k, v, g, T=T, causal=True, n_sink=1, window=2)
    b = oracle.softmax_anchor(q, k[:, :, perm], v[:, :, perm], g, T=T, causal=True, n_sink=1,
                              window=2)
    assert close(a, b, 1e-13)


def test_bf16_inputs_are_read_exactly():
    rng = np.random.default_rng(9)
    q, k, v, g = rand(rng, 1, 2, 3, 3, 4, 8)
    bits = [(x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for x in (q, k, v, g)]
    vals = [oracle.bf16_to_f64(b) for b in bits]
    a = oracle.softmax_anchor(*bits, T=4, causal=True, n_sink=1, window=2)
    b = oracle.softmax_anchor(*vals, T=4, causal=True, n_sink=1, window=2)
    assert np.array_equal(a, b)
