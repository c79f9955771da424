"""GPU parity of the frame-wise Gated DeltaNet (gla_gdn_framecausal, through the
C ABI) against the fp64 oracle (oracle.gdn, pinned in test_oracle_gdn.py).

Bar: slab-normalised error of o at most 1e-4 (float32) and 2e-2 (bfloat16 with
fp32 accumulation); the carried state by max|dS| / max|S| <= 1e-4.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
import oracle
from gated_linear_attention_fwd_amd import synth
from gla_testutil import TOL, max_abs_over_max, slab_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
STATE_TOL = 1e-4
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_worked_example_d1.json")


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


def gdn_inputs(B, H, F, T, d, dtype, seed):
    """q, k, v as the synthetic recipe draws them; beta = sigmoid(N(0, 1)) per
    token; gamma as the recipe's frame decays."""
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=seed)
    rng = np.random.default_rng(seed + 1)
    x["beta"] = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, F * T))))).astype(np.float32)
    return x


def report(name, **errs):
    print(name, " ".join("%s=%.3e" % kv for kv in errs.items()), flush=True)


CASES = [
    # (dtype, B, H, d, F, T, carry)
    ("f32", 1, 2, 16, 4, 16, False),
    ("f32", 1, 3, 64, 3, 37, True),
    ("bf16", 1, 4, 64, 5, 256, True),
    ("bf16", 2, 2, 32, 6, 61, True),
    ("bf16", 1, 2, 128, 3, 100, True),
    ("bf16", 1, 3, 16, 4, 33, False),
    ("bf16", 1, 2, 64, 1, 40, True),     # a single frame
    ("bf16", 1, 2, 64, 2, 300, False),   # three parts per frame, ragged last part
    ("bf16", 1, 2, 128, 4, 520, True),   # five parts per frame at d = 128
    ("bf16", 1, 2, 64, 70, 24, True),    # scan in chunks of 32 frames, a ragged last chunk
    ("bf16", 1, 2, 32, 64, 16, True),    # exactly two chunks
    ("bf16", 1, 1, 128, 65, 20, True),   # a last chunk of one frame
    ("f32", 1, 2, 64, 66, 8, True),      # the vector-ALU scan at the same length
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-B%dH%d-d%d-F%dT%d-carry%d" % c)
def test_gdn(case, path):
    dtype, B, H, d, F, T, carry = case
    x = gdn_inputs(B, H, F, T, d, dtype, seed=600 + d + T)
    S_in = np.random.default_rng(9).standard_normal((B, H, d, d)).astype(np.float32) \
        if carry else None
    o, S = gla.gla_gdn_framecausal(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["beta"]),
                                   dev(x["gamma"]), None if S_in is None else dev(S_in),
                                   return_state=True)
    ro, rS = oracle.gdn(x["q"], x["k"], x["v"], x["beta"], x["gamma"], S_in=S_in)
    e_o = slab_rel_err(f64(o), ro)
    e_S = max_abs_over_max(S.cpu().numpy(), rS)
    report("gdn %s %s" % (case, path), o=e_o, S=e_S)
    assert e_o <= TOL[dtype] and e_S <= STATE_TOL
    # the state-only call commits the same state, bit for bit
    S2 = gla.gla_gdn_framecausal(None, dev(x["k"]), dev(x["v"]), dev(x["beta"]), dev(x["gamma"]),
                                 None if S_in is None else dev(S_in))
    assert torch.equal(S2, S)


def test_gdn_worked_example_padded():
    """The hand-worked d = 1 example, zero-padded to d = 16 (the padding never
    interacts with feature 0): o and S_out as derived by hand."""
    g = json.load(open(GOLDEN))
    d, N = 16, 4

    def pad(a):
        a = np.array(a, np.float32)
        out = np.zeros(a.shape[:-1] + (d,), np.float32)
        out[..., :1] = a
        return out
    q, k, v = pad(g["q"]), pad(g["k"]), pad(g["v"])
    S_in = np.zeros((1, 1, d, d), np.float32)
    S_in[0, 0, 0, 0] = g["S_in"][0][0][0][0]
    o, S = gla.gla_gdn_framecausal(dev(q), dev(k), dev(v), dev(np.array(g["beta"], np.float32)),
                                   dev(np.array(g["gamma"], np.float32)), dev(S_in),
                                   key_scale=g["key_scale"], return_state=True)
    want = np.zeros((1, 1, N, d))
    want[..., :1] = np.array(g["o"])
    assert np.allclose(o.cpu().numpy(), want, atol=1e-6)
    assert np.allclose(S.cpu().numpy(), 0.0, atol=1e-6)


def test_gdn_block_split_with_carry():
    B, H, d, F, T = 1, 4, 64, 7, 96
    x = gdn_inputs(B, H, F, T, d, "bf16", seed=31)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "gamma")}
    o, S = gla.gla_gdn_framecausal(t["q"], t["k"], t["v"], t["beta"], t["gamma"],
                                   return_state=True)
    outs, Sc = [], None
    for f0, nf in ((0, 3), (3, 4)):
        sl = slice(f0 * T, (f0 + nf) * T)
        ob, Sc = gla.gla_gdn_framecausal(t["q"][:, :, sl].contiguous(), t["k"][:, :, sl].contiguous(),
                                         t["v"][:, :, sl].contiguous(),
                                         t["beta"][:, :, sl].contiguous(),
                                         t["gamma"][:, :, f0:f0 + nf].contiguous(), Sc,
                                         key_scale=1 / np.sqrt(d * T), return_state=True)
        outs.append(ob)
    e_o = slab_rel_err(f64(torch.cat(outs, dim=2)), f64(o))
    e_S = max_abs_over_max(Sc.cpu().numpy(), S.cpu().numpy().astype(np.float64))
    report("gdn block split", o=e_o, S=e_S)
    assert e_o <= TOL["bf16"] and e_S <= STATE_TOL


def test_gdn_no_writes():
    """beta = 0: o_t = (prod gamma) S_in^T q_t."""
    B, H, d, F, T = 1, 2, 32, 3, 40
    x = gdn_inputs(B, H, F, T, d, "f32", seed=4)
    S_in = np.random.default_rng(2).standard_normal((B, H, d, d)).astype(np.float32)
    o = gla.gla_gdn_framecausal(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                                torch.zeros((B, H, F * T), device=DEV), dev(x["gamma"]),
                                dev(S_in))
    w = np.repeat(np.cumprod(x["gamma"].astype(np.float64), axis=-1), T, axis=-1)[..., None]
    want = np.einsum("bhnd,bhde->bhne", x["q"].astype(np.float64), S_in.astype(np.float64)) * w
    assert slab_rel_err(o.cpu().numpy(), want) <= TOL["f32"]


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 64), ("bf16", 128)])
def test_gdn_no_tokens(dtype, d):
    """T = 0: every frame only decays the state, S_out = (prod gamma) S_in."""
    B, H, F = 1, 2, 3
    rng = np.random.default_rng(d)
    S_in = rng.standard_normal((B, H, d, d)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.0, (B, H, F)).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    e = torch.empty((B, H, 0, d), dtype=tdt, device=DEV)
    o, S = gla.gla_gdn_framecausal(e, e, e, torch.empty((B, H, 0), device=DEV), dev(gamma),
                                   dev(S_in), key_scale=0.5, return_state=True)
    want = S_in.astype(np.float64) * np.prod(gamma.astype(np.float64), axis=-1)[..., None, None]
    assert o.numel() == 0
    assert max_abs_over_max(S.cpu().numpy(), want) <= STATE_TOL


def test_gdn_720p_60s_sampled_heads():
    """The 720p/60s shape (B=1, H=32, d=64, 241 frames of 920 tokens, bf16) with
    beta = sigmoid of a device normal draw; two heads against the oracle."""
    w = synth.WORKLOADS[4]
    xd = synth.device_inputs(w, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(w.seed * 1000 + 11)
    beta = torch.sigmoid(torch.randn((w.B, w.H, w.N), generator=gen, device=DEV))
    o, S = gla.gla_gdn_framecausal(xd["q"], xd["k"], xd["v"], beta, xd["gamma"],
                                   return_state=True)
    torch.cuda.synchronize()
    for h in (0, 17):
        sel = slice(h, h + 1)
        ro, rS = oracle.gdn(host(xd["q"][:, sel]), host(xd["k"][:, sel]), host(xd["v"][:, sel]),
                            beta[:, sel].cpu().numpy(), xd["gamma"][:, sel].cpu().numpy())
        e_o = slab_rel_err(f64(o[:, sel]), ro)
        e_S = max_abs_over_max(S[:, sel].cpu().numpy(), rS)
        report("gdn 720p/60s head %d" % h, o=e_o, S=e_S)
        assert e_o <= TOL["bf16"] and e_S <= STATE_TOL
