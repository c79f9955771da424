"""Past 2^31 elements per tensor: 64-bit offsets everywhere.

B=1, H=2, 18500 frames of 920 tokens, d=64, bf16: 2.18e9 elements per tensor
(4.3 GB). With every frame decay gamma_f = 0 each frame is independent of the
others (S_f is the frame's own sum), so sampled frames at the start, middle
and end of the slabs are checked against the fp64 oracle run on that frame
alone; the softmax anchor gets the same independence from a window of one
frame and no sinks."""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
import oracle
from gla_testutil import TOL, slab_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, H, T, D = 1, 2, 920, 64
F = 18500
N = F * T
FRAMES = (0, F // 2, F - 1)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert B * H * N * D > 2 ** 31
    gla.load_library()
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def draw(names, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    out = {}
    for n in names:
        out[n] = torch.randn((B, H, N, D), generator=gen, device=DEV, dtype=torch.bfloat16)
    return out


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def frame(t, h, f):
    return host(t[:, h:h + 1, f * T:(f + 1) * T])


def f64(t) -> np.ndarray:
    return oracle.bf16_to_f64(t) if t.dtype == np.uint16 else t.astype(np.float64)


def test_forward_framecausal():
    x = draw("qkvg", seed=101)
    gamma = torch.zeros((B, H, F), device=DEV)
    o = gla.gla_fwd_framecausal(x["q"], x["k"], x["v"], x["g"], gamma)
    torch.cuda.synchronize()
    for h in range(H):
        for f in FRAMES:
            fx = {n: frame(x[n], h, f) for n in "qkvg"}
            ref, _, _ = oracle.recurrent(oracle.FRAMECAUSAL, fx["q"], fx["k"], fx["v"], fx["g"],
                                         np.zeros((1, 1, 1)))
            assert slab_rel_err(f64(frame(o, h, f)), ref) <= TOL["bf16"], (h, f)


def test_backward_framecausal():
    x = draw(["q", "k", "v", "g", "dO"], seed=102)
    gamma = torch.zeros((B, H, F), device=DEV)
    got = gla.gla_bwd_framecausal(x["q"], x["k"], x["v"], x["g"], gamma, x["dO"])
    torch.cuda.synchronize()
    for h in range(H):
        for f in FRAMES:
            fx = {n: frame(x[n], h, f) for n in ("q", "k", "v", "g", "dO")}
            ref = oracle.backward(oracle.FRAMECAUSAL, fx["q"], fx["k"], fx["v"], fx["g"], fx["dO"],
                                  gamma=np.zeros((1, 1, 1)))
            for n in ("dq", "dk", "dv", "dg"):
                assert slab_rel_err(f64(frame(got[n], h, f)), ref[n]) <= TOL["bf16"], (n, h, f)


def test_gated_deltanet():
    x = draw("qkv", seed=103)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(104)
    beta = torch.sigmoid(torch.randn((B, H, N), generator=gen, device=DEV))
    gamma = torch.zeros((B, H, F), device=DEV)
    o = gla.gla_gdn_framecausal(x["q"], x["k"], x["v"], beta, gamma)
    torch.cuda.synchronize()
    for h in range(H):
        for f in FRAMES:
            fx = {n: frame(x[n], h, f) for n in "qkv"}
            b = beta[:, h:h + 1, f * T:(f + 1) * T].cpu().numpy()
            ref, _ = oracle.gdn(fx["q"], fx["k"], fx["v"], b, np.zeros((1, 1, 1)),
                                key_scale=1.0 / np.sqrt(D * T))
            assert slab_rel_err(f64(frame(o, h, f)), ref) <= TOL["bf16"], (h, f)


def test_softmax_anchor():
    x = draw("qkvg", seed=105)
    o = gla.gla_softmax_anchor(x["q"], x["k"], x["v"], x["g"], T=T, n_sink=0, window=1)
    torch.cuda.synchronize()
    for h in range(H):
        for f in FRAMES:
            fx = {n: frame(x[n], h, f) for n in "qkvg"}
            ref = oracle.softmax_anchor(fx["q"], fx["k"], fx["v"], fx["g"], T=T, window=1)
            assert slab_rel_err(f64(frame(o, h, f)), ref) <= TOL["bf16"], (h, f)
