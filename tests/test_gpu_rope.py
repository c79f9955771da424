"""GPU parity of the strided layouts and the fused 3D rotary positions
(gla_*_ex entry points) against the fp64 oracle.

Reading under test (the SANA-Video ICLR 2026 oral talk adds 3D RoPE to the
linear attention without placing it): RoFormer's rotary linear attention --
turned phi(q), phi(k) in the numerator, unturned in the normaliser. The oracle
side is oracle.rope_recurrent, pinned in test_oracle_rope.py.

Bar as in test_gpu_parity.py: slab-normalised error of o <= 1e-4 (float32),
2e-2 (bfloat16 with fp32 accumulation); states max|dS| / max|S| <= 1e-4. Layout
changes alone must not change a single bit. (The matrix-core kernels feed the
turned features to the MFMAs as bf16 hi + lo pairs, so the turns cost no
precision beyond fp32: a single bf16 rounding of them would put the state
~1.5e-3 off and o past 2e-2 at 241 frames.)
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
STATE_TOL = 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.load_library()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=["auto", "valu"])
def path(request, monkeypatch):
    """Run with the default kernel choice and with the vector-ALU kernels forced."""
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


def bnhd(x: np.ndarray) -> torch.Tensor:
    """[B, H, N, d] values stored as [B, N, H, d]; returns the [B, H, N, d] view."""
    return dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).transpose(1, 2)


def fused(q, k, v):
    """q, k, v stored as one [B, N, 3, H, d] tensor; returns the three views."""
    X = dev(np.ascontiguousarray(np.stack([q, k, v], axis=0).transpose(1, 3, 0, 2, 4)))
    return tuple(X[:, :, i].transpose(1, 2) for i in range(3))


def sections(d: int):
    """(dim_t, dim_h, dim_w): h and w take 2 * (d // 6) features each, t the rest."""
    s = 2 * (d // 6)
    return d - 2 * s, s, s


def rope_for(gh, gw, d, frame_offset=0, theta=10000.0, dims=None):
    dt_, dh, dw = dims or sections(d)
    return dict(grid_h=gh, grid_w=gw, frame_offset=frame_offset, dim_t=dt_, dim_h=dh, dim_w=dw,
                theta=theta)


def check_state(S, rS):
    """max|dS| / max|S|."""
    return max_abs_over_max(S.detach().cpu().numpy(), rS)


def report(name, **errs):
    print(name, " ".join("%s=%.3e" % kv for kv in errs.items()), flush=True)


# ---------------------------------------------------------------- layouts only

@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 32), ("bf16", 128)])
def test_strided_layouts_bit_identical(dtype, d, path):
    """[B, N, H, d] views and a fused [B, N, 3, H, d] projection give the very
    bits of the contiguous call (both modes, carried state included)."""
    B, H, F, T = 2, 3, 3, 200
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=71 + d)
    q, k, v, g = (dev(x[n]) for n in "qkvg")
    gamma = dev(x["gamma"])
    rng = np.random.default_rng(5)
    S_in = dev(rng.standard_normal((B, H, d, d)).astype(np.float32))
    z_in = dev(np.abs(rng.standard_normal((B, H, d))).astype(np.float32))
    o_ref, S_ref, z_ref = gla.gla_fwd_framecausal(q, k, v, g, gamma, S_in, z_in, return_state=True)
    ob_ref = gla.gla_fwd_bidir(q, k, v, g)

    qs, ks, vs = fused(x["q"], x["k"], x["v"])
    gs = bnhd(x["g"])
    out = torch.empty((B, F * T, H, d), dtype=q.dtype, device=DEV).transpose(1, 2)
    o, S, z = gla.gla_fwd_framecausal_ex(qs, ks, vs, gs, gamma, S_in, z_in, out=out,
                                         return_state=True)
    assert o.data_ptr() == out.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref) and torch.equal(z, z_ref)
    ob = gla.gla_fwd_bidir_ex(bnhd(x["q"]), bnhd(x["k"]), bnhd(x["v"]), gs)
    assert torch.equal(ob, ob_ref)
    S2, z2 = gla.gla_state_carry_ex(ks, vs, gamma, S_in, z_in)
    assert torch.equal(S2, S_ref) and torch.equal(z2, z_ref)


def test_broadcast_gate_over_heads():
    """A zero head stride (one gate shared by every head) is a valid input view."""
    B, H, F, T, d = 1, 4, 2, 96, 64
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=9)
    g1 = dev(x["g"][:, :1])
    g_b = g1.expand(B, H, F * T, d)
    assert g_b.stride(1) == 0
    q, k, v = (dev(x[n]) for n in "qkv")
    gamma = dev(x["gamma"])
    o = gla.gla_fwd_framecausal_ex(q, k, v, g_b, gamma)
    o_ref = gla.gla_fwd_framecausal(q, k, v, g_b.contiguous(), gamma)
    assert torch.equal(o, o_ref)


# ------------------------------------------------------------- rotary positions

ROPE_CASES = [
    # (dtype, d, grid_h, grid_w, F, frames per kv group or None, sections or None)
    ("bf16", 64, 5, 7, 4, None, None),         # ragged 35-token frames
    ("bf16", 64, 12, 20, 3, None, None),       # 240-token frames: several kv parts
    ("bf16", 64, 6, 9, 7, 3, None),            # groups of 3 frames with a carry chain
    ("bf16", 32, 4, 10, 5, 2, None),
    ("bf16", 128, 8, 8, 3, None, None),
    ("bf16", 128, 8, 8, 3, 2, None),          # d = 128 asked for frame pairs: one frame per group
    ("bf16", 64, 4, 6, 3, None, (0, 32, 32)),  # no temporal section
    ("bf16", 64, 4, 6, 3, None, (64, 0, 0)),   # temporal only
    ("bf16", 16, 3, 5, 3, None, None),         # vector-ALU kernels (no matrix-core d = 16)
    ("f32", 64, 5, 7, 4, None, None),
    ("f32", 128, 3, 4, 2, None, None),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "%s-d%d-%dx%d-F%d-G%s-%s" % c)
def test_rope_framecausal(case, path, monkeypatch):
    dtype, d, gh, gw, F, G, dims = case
    if G:
        monkeypatch.setenv("GLA_FRAMES_PER_GROUP", str(G))
    B, H, T = 1, 3, gh * gw
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=400 + d + F)
    rope = rope_for(gh, gw, d, frame_offset=5, dims=dims)
    rng = np.random.default_rng(17)
    S_in = rng.standard_normal((B, H, d, d)).astype(np.float32)
    z_in = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
    qs, ks, vs = fused(x["q"], x["k"], x["v"])
    o, S, z = gla.gla_fwd_framecausal_ex(qs, ks, vs, bnhd(x["g"]), dev(x["gamma"]), dev(S_in),
                                         dev(z_in), rope=rope, return_state=True)
    ro, rS, rz = oracle.rope_recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                       x["gamma"], S_in=S_in, z_in=z_in, rope=rope)
    e_o = slab_rel_err(f64(o), ro)
    e_S = check_state(S, rS)
    e_z = max_abs_over_max(z.cpu().numpy(), rz)
    report("rope framecausal %s %s" % (case, path), o=e_o, S=e_S, z=e_z)
    assert e_o <= TOL[dtype]
    assert e_S <= STATE_TOL and e_z <= STATE_TOL
    # the state commit agrees with the forward pass bit for bit
    S2, z2 = gla.gla_state_carry_ex(ks, vs, dev(x["gamma"]), dev(S_in), dev(z_in), rope=rope)
    assert torch.equal(S2, S) and torch.equal(z2, z)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("bf16", 16)])
def test_rope_bidir(dtype, d, path):
    B, H, gh, gw, F = 1, 2, 6, 10, 4
    T = gh * gw
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=500 + d)
    rope = rope_for(gh, gw, d, frame_offset=2)
    o = gla.gla_fwd_bidir_ex(bnhd(x["q"]), bnhd(x["k"]), bnhd(x["v"]), bnhd(x["g"]), rope=rope)
    ro = oracle.rope_recurrent(oracle.BIDIR, x["q"], x["k"], x["v"], x["g"], F=F, T=T,
                               rope=rope)[0]
    e = slab_rel_err(f64(o), ro)
    report("rope bidir %s d=%d %s" % (dtype, d, path), o=e)
    assert e <= TOL[dtype]


def test_rope_stream_in_blocks():
    """Frames streamed in blocks, each passing its first frame as frame_offset
    and carrying (S, z): the outputs and final state of the one-shot call."""
    B, H, gh, gw, d = 1, 4, 8, 12, 64
    T, F = gh * gw, 9
    x = synth.random_inputs(B, H, F, T, d, "bf16", seed=77)
    q, k, v, g = (dev(x[n]) for n in "qkvg")
    gamma = dev(x["gamma"])
    o1, S1, z1 = gla.gla_fwd_framecausal_ex(q, k, v, g, gamma, rope=rope_for(gh, gw, d),
                                            return_state=True)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device=DEV)
    z = torch.zeros((B, H, d), dtype=torch.float32, device=DEV)
    outs = []
    for f0, nf in ((0, 4), (4, 3), (7, 2)):
        sl = slice(f0 * T, (f0 + nf) * T)
        o, S, z = gla.gla_fwd_framecausal_ex(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, sl],
                                             gamma[:, :, f0:f0 + nf].contiguous(), S, z,
                                             rope=rope_for(gh, gw, d, frame_offset=f0),
                                             return_state=True)
        outs.append(o)
    o2 = torch.cat(outs, dim=2)
    e_o = slab_rel_err(f64(o2), f64(o1))
    e_S = max_abs_over_max(S.cpu().numpy(), S1.cpu().numpy().astype(np.float64))
    report("rope stream in blocks", o=e_o, S=e_S)
    assert e_o <= TOL["bf16"] and e_S <= STATE_TOL
    ro = oracle.rope_recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"], x["gamma"],
                               rope=rope_for(gh, gw, d))[0]
    assert slab_rel_err(f64(o2), ro) <= TOL["bf16"]


def test_rope_changes_the_result():
    """With positions the output differs from the plain call by far more than
    the bf16 tolerance (the turns are applied at all)."""
    B, H, gh, gw, F, d = 1, 2, 5, 8, 3, 64
    x = synth.random_inputs(B, H, F, gh * gw, d, "bf16", seed=3)
    q, k, v, g = (dev(x[n]) for n in "qkvg")
    gamma = dev(x["gamma"])
    a = gla.gla_fwd_framecausal_ex(q, k, v, g, gamma, rope=rope_for(gh, gw, d, theta=3.0))
    b = gla.gla_fwd_framecausal(q, k, v, g, gamma)
    assert slab_rel_err(f64(a), f64(b)) > 10 * TOL["bf16"]


def test_rope_720p_60s_fused_layout_sampled_heads():
    """The 720p/60s shape (B=1, H=32, d=64, 241 frames of 23 x 40 tokens, bf16)
    read from a fused [B, N, 3, H, d] projection with positions, in the launch
    configuration the benchmark times; three heads against the oracle."""
    w = synth.WORKLOADS[4]
    assert (w.T, w.d) == (23 * 40, 64)
    xd = synth.device_inputs(w, DEV)
    q, k, v, g, gamma = (xd.pop(n) for n in ("q", "k", "v", "g", "gamma"))
    X = torch.stack([q, k, v], dim=0).permute(1, 3, 0, 2, 4).contiguous()  # [B, N, 3, H, d]
    del q, k, v
    qs, ks, vs = (X[:, :, i].transpose(1, 2) for i in range(3))
    rope = rope_for(23, 40, w.d)
    out = torch.empty((w.B, w.N, w.H, w.d), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    o, S, z = gla.gla_fwd_framecausal_ex(qs, ks, vs, g, gamma, rope=rope, out=out,
                                         return_state=True)
    torch.cuda.synchronize()
    for h in (0, 13, 31):
        sel = slice(h, h + 1)
        xs = {n: host(t[:, sel]) for n, t in zip("qkvg", (qs, ks, vs, g))}
        xs["gamma"] = host(gamma[:, sel])
        ro, rS, _ = oracle.rope_recurrent(oracle.FRAMECAUSAL, xs["q"], xs["k"], xs["v"], xs["g"],
                                          xs["gamma"], rope=rope, eps=w.eps)
        e_o = slab_rel_err(f64(o[:, sel]), ro)
        e_S = check_state(S[:, sel], rS)
        report("rope 720p/60s head %d" % h, o=e_o, S=e_S)
        assert e_o <= TOL["bf16"] and e_S <= STATE_TOL
