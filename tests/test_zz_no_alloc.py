"""gla_fwd_framecausal_noalloc, the frame-causal forward whose workspace is the
library's static device scratch, called through the C ABI: its outputs equal
those of gla_fwd_framecausal with a caller's workspace bit for bit (the same
kernels and plan), and so meet the parity bar that test_gpu_parity.py checks
for that call against the oracle. Two calls in a row share the scratch, the
second on smaller sizes, as do the matrix-core (bf16) and vector-ALU (fp32)
kernels; a third call checks the larger sizes again over the smaller call's
leftovers."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gated_linear_attention_fwd_amd as gla
import oracle
from gated_linear_attention_fwd_amd import synth

from gla_testutil import TOL, slab_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.load_library()
    yield
    torch.cuda.synchronize()


def inputs(B, H, F, T, d, dtype, seed):
    x = synth.random_inputs(B, H, F, T, d, dtype, seed=seed, scale_qkv=True, gamma_mu=3.0)
    if dtype == "bf16":
        t = {n: torch.from_numpy(x[n].view(np.int16)).to(DEV).view(torch.bfloat16) for n in "qkvg"}
    else:
        t = {n: torch.from_numpy(x[n]).to(DEV) for n in "qkvg"}
    t["gamma"] = torch.from_numpy(x["gamma"]).to(DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed + 100)
    t["S_in"] = torch.randn((B, H, d, d), generator=gen, device=DEV)
    t["z_in"] = torch.rand((B, H, d), generator=gen, device=DEV)
    return x, t


def c_noalloc(t, o, S_out, z_out, eps=1e-6):
    """The entry point through ctypes, on the current stream."""
    lib = gla.load_library()
    B, H, N, d = t["q"].shape
    F = t["gamma"].shape[-1]
    vp = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    dt = 1 if t["q"].dtype == torch.bfloat16 else 0
    st = lib.gla_fwd_framecausal_noalloc(
        vp(t["q"]), vp(t["k"]), vp(t["v"]), vp(t["g"]), vp(t["gamma"]), vp(t["S_in"]),
        vp(t["z_in"]), vp(o), vp(S_out), vp(z_out), B, H, F, N // F, d, dt, ctypes.c_float(eps),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.gla_last_error().decode()


def run_both(shape, dtype, seed):
    x, t = inputs(*shape, dtype, seed)
    B, H, F, T, d = shape
    o = torch.empty_like(t["q"])
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    c_noalloc(t, o, S, z)
    ref_o, ref_S, ref_z = gla.gla_fwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"],
                                                  t["S_in"], t["z_in"], return_state=True)
    torch.cuda.synchronize()
    return x, t, (o, S, z), (ref_o, ref_S, ref_z)


@pytest.mark.parametrize("dtype,shapes", [
    ("bf16", [(1, 4, 5, 300, 64), (1, 2, 3, 100, 64)]),
    ("f32", [(1, 3, 4, 64, 16), (1, 2, 2, 40, 16)]),
])
def test_noalloc_equals_workspace_call(dtype, shapes):
    print("noalloc: %s, sizes %s then %s" % (dtype, shapes[0], shapes[1]), flush=True)
    for i, shape in enumerate(shapes + shapes[:1]):
        x, t, got, want = run_both(shape, dtype, seed=40 + i)
        for a, b, n in zip(got, want, ("o", "S_out", "z_out")):
            assert torch.equal(a, b), (shape, n)
        if i == 1:  # the smaller call: also the parity bar against the oracle
            ro, rS, _ = oracle.recurrent(oracle.FRAMECAUSAL, x["q"], x["k"], x["v"], x["g"],
                                         x["gamma"], S_in=t["S_in"].cpu().numpy(),
                                         z_in=t["z_in"].cpu().numpy())
            o = got[0]
            o64 = (oracle.bf16_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
                   if dtype == "bf16" else o.cpu().numpy().astype(np.float64))
            assert slab_rel_err(o64, ro) <= TOL[dtype]
            assert np.max(np.abs(got[1].cpu().numpy() - rS)) <= 1e-4 * np.max(np.abs(rS))


def test_noalloc_python_binding_and_refusal():
    """The binding of the same name, and a size beyond the scratch refused
    with GLA_ERR_WORKSPACE before any launch."""
    x, t = inputs(1, 2, 3, 100, 64, "bf16", 50)
    o = torch.empty_like(t["q"])
    gla.gla_fwd_framecausal_noalloc(t["q"], t["k"], t["v"], t["g"], t["gamma"], o,
                                    t["S_in"], t["z_in"])
    want = gla.gla_fwd_framecausal(t["q"], t["k"], t["v"], t["g"], t["gamma"], t["S_in"],
                                   t["z_in"])
    torch.cuda.synchronize()
    assert torch.equal(o, want)
    lib = gla.load_library()
    st = lib.gla_fwd_framecausal_noalloc(
        *(ctypes.c_void_p(t[n].data_ptr()) for n in ("q", "k", "v", "g", "gamma")), None, None,
        ctypes.c_void_p(o.data_ptr()), None, None, 1, 128, 241, 920, 64, 1,
        ctypes.c_float(1e-6), None)
    assert st == 5  # GLA_ERR_WORKSPACE
