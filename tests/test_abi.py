"""C-ABI checks that need no GPU: the library loads, exports what include/gla.h
declares, sizes its workspace as documented and rejects bad arguments on the
host before anything is launched (every call below fails validation or has no
work, so no HIP call is made)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import gated_linear_attention_fwd_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, VALUE, HIP, ALIAS = range(9)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.library_path()):
        from gated_linear_attention_fwd_amd import build
        build.build_library()
    return gla.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(gla_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("gla_fwd_bidir", "gla_fwd_framecausal", "gla_state_carry",
              "gla_fwd_bidir_workspace", "gla_fwd_framecausal_workspace",
              "gla_state_carry_workspace", "gla_status_string", "gla_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(9):
        assert lib.gla_status_string(s).decode()
    assert lib.gla_status_string(99).decode() == "unknown status"
    assert lib.gla_version() == 10600


def test_workspace_sizes(lib):
    # 720p/60s: one part per frame, a state of d*d + d floats per (slab, frame),
    # plus one carried state per group of 8 frames (31 groups of 241 frames)
    E = 64 * 64 + 64
    assert gla.gla_fwd_framecausal_workspace(1, 32, 241, 920, 64) == (32 * 241 + 32 * 31) * E * 4
    assert gla.gla_state_carry_workspace(1, 32, 241, 920, 64) == (32 * 241 + 32 * 31) * E * 4
    # d = 128 pairs frames from 1536 frames on (a carried state per pair of the
    # 30-frame block's 15), and below that runs one frame per group, the scan
    # completing each state in place (480 frames: two parts per frame)
    E2 = 128 * 128 + 128
    assert gla.gla_fwd_framecausal_workspace(2, 40, 30, 920, 128) == (80 * 30 + 80 * 15) * E2 * 4
    assert gla.gla_fwd_framecausal_workspace(1, 16, 30, 920, 128) == 16 * 30 * 2 * E2 * 4
    # small problems are cut into parts to fill the GPU: the size grows accordingly
    small = gla.gla_fwd_framecausal_workspace(1, 8, 5, 256, 64)
    assert small > 8 * 5 * 4160 * 4 and small % 256 == 0
    assert gla.gla_fwd_bidir_workspace(1, 32, 19320, 64) % (4160 * 4) == 0
    assert gla.gla_fwd_bidir_workspace(1, 32, 19320, 64) > 32 * 4160 * 4
    # empty and invalid sizes need nothing
    assert gla.gla_fwd_framecausal_workspace(0, 32, 241, 920, 64) == 0
    assert gla.gla_fwd_bidir_workspace(1, 1, 0, 64) == 0
    assert gla.gla_fwd_framecausal_workspace(1, 1, -1, 4, 64) == 0


FAKE = 0x10000  # an aligned non-NULL address; never dereferenced on these paths


def p(x):
    return ctypes.c_void_p(x) if x else None


def bidir(lib, q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, g=FAKE + 0x3000000,
          o=FAKE + 0x4000000, B=1, H=1, N=64, d=64, dt=BF16, eps=1e-6, ws=FAKE + 0x8000000,
          wsb=1 << 30):
    return lib.gla_fwd_bidir(p(q), p(k), p(v), p(g), p(o), B, H, N, d, dt, eps, p(ws), wsb, None)


def framecausal(lib, q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, g=FAKE + 0x3000000,
                gamma=FAKE + 0x5000000, S_in=None, z_in=None, o=FAKE + 0x4000000, S_out=None,
                z_out=None, B=1, H=1, F=2, T=32, d=64, dt=BF16, eps=1e-6, ws=FAKE + 0x8000000,
                wsb=1 << 30):
    return lib.gla_fwd_framecausal(p(q), p(k), p(v), p(g), p(gamma), p(S_in), p(z_in), p(o),
                                   p(S_out), p(z_out), B, H, F, T, d, dt, eps, p(ws), wsb, None)


def carry(lib, k=FAKE, v=FAKE + 0x1000000, gamma=FAKE + 0x5000000, S_in=None, z_in=None,
          S_out=FAKE + 0x6000000, z_out=FAKE + 0x7000000, B=1, H=1, F=2, T=32, d=64, dt=BF16,
          ws=FAKE + 0x8000000, wsb=1 << 30):
    return lib.gla_state_carry(p(k), p(v), p(gamma), p(S_in), p(z_in), p(S_out), p(z_out), B, H,
                               F, T, d, dt, p(ws), wsb, None)


def test_bidir_validation(lib):
    assert bidir(lib, d=48) == UNSUP
    assert bidir(lib, d=256) == UNSUP
    assert bidir(lib, dt=7) == UNSUP
    assert bidir(lib, B=-1) == SHAPE
    assert bidir(lib, N=-5) == SHAPE
    assert bidir(lib, eps=-1.0) == VALUE
    assert bidir(lib, eps=float("nan")) == VALUE
    assert bidir(lib, eps=float("inf")) == VALUE
    assert bidir(lib, q=0) == NULL
    assert bidir(lib, o=0) == NULL
    assert bidir(lib, k=FAKE + 0x1000008) == ALIGN
    assert bidir(lib, ws=0) == WS
    assert bidir(lib, wsb=16) == WS
    assert bidir(lib, ws=FAKE + 0x8000010) == ALIGN
    assert bidir(lib, o=FAKE + 0x100) == ALIAS  # o overlaps q
    assert bidir(lib, ws=FAKE + 0x4000000) == ALIAS  # workspace overlaps o
    assert "overlaps" in lib.gla_last_error().decode()
    # empty problems are valid and launch nothing
    assert bidir(lib, N=0) == OK
    assert bidir(lib, B=0) == OK
    assert bidir(lib, H=0, q=0, k=0, v=0, g=0, o=0) == OK


def test_framecausal_validation(lib):
    assert framecausal(lib, d=8) == UNSUP
    assert framecausal(lib, F=-1) == SHAPE
    assert framecausal(lib, T=-1) == SHAPE
    assert framecausal(lib, gamma=0) == NULL
    assert framecausal(lib, S_in=FAKE + 0x6000000) == NULL  # S_in without z_in
    assert framecausal(lib, z_out=FAKE + 0x7000000) == NULL  # z_out without S_out
    assert framecausal(lib, g=0) == NULL
    assert framecausal(lib, gamma=FAKE + 0x5000002) == ALIGN
    assert framecausal(lib, S_out=FAKE + 0x6000004, z_out=FAKE + 0x7000000) == ALIGN
    assert framecausal(lib, eps=-1e-3) == VALUE
    assert framecausal(lib, wsb=0) == WS
    assert framecausal(lib, S_out=FAKE, z_out=FAKE + 0x7000000) == ALIAS  # S_out overlaps q
    assert framecausal(lib, S_in=FAKE + 0x6000000, z_in=FAKE + 0x6000000 + 64,
                       S_out=FAKE + 0x6000000 + 1024, z_out=FAKE + 0x7000000) == ALIAS
    assert framecausal(lib, B=0) == OK
    assert "gamma" in (framecausal(lib, gamma=0) and lib.gla_last_error().decode())


def test_state_carry_validation(lib):
    assert carry(lib, S_out=0, z_out=0) == NULL
    assert carry(lib, d=100) == UNSUP
    assert carry(lib, k=0) == NULL
    assert carry(lib, wsb=8) == WS
    assert carry(lib, S_out=FAKE, z_out=FAKE + 0x7000000) == ALIAS
    assert carry(lib, H=0) == OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 32, 16)
    with pytest.raises(ValueError, match="GPU"):
        gla.gla_fwd_bidir(x, x, x, x)
    with pytest.raises(TypeError):
        gla.gla_fwd_bidir(x.double(), x.double(), x.double(), x.double())


def tview(data, sb, sh, sn):
    return ctypes.byref(gla._Tensor(data or None, sb, sh, sn))


def rope3d(gh=4, gw=8, off=0, dt_=16, dh=24, dw=24, theta=10000.0):
    return ctypes.byref(gla.Rope3D(gh, gw, dt_, dh, dw, theta, off))


def fc_ex(lib, q=None, k=None, v=None, g=None, o=None, rope="default", B=1, H=2, F=2, T=32,
          d=64, dt=BF16, ws=FAKE + 0x8000000, wsb=1 << 30):
    """framecausal_ex on [B][N][H][d] views (contiguous strides of that layout)"""
    N = F * T
    lay = (N * H * d, d, H * d)
    q = q or tview(FAKE, *lay)
    k = k or tview(FAKE + 0x1000000, *lay)
    v = v or tview(FAKE + 0x2000000, *lay)
    g = g or tview(FAKE + 0x3000000, *lay)
    o = o or tview(FAKE + 0x4000000, *lay)
    r = rope3d() if rope == "default" else rope
    return lib.gla_fwd_framecausal_ex(q, k, v, g, p(FAKE + 0x5000000), None, None, o, None, None,
                                      B, H, F, T, d, dt, 1e-6, r, p(ws), wsb, None)


def test_ex_validation(lib):
    N, H, d = 64, 2, 64
    # rotary parameters
    assert fc_ex(lib, rope=rope3d(gh=3)) == SHAPE  # grid does not hold T tokens
    assert fc_ex(lib, rope=rope3d(dt_=15, dh=25)) == SHAPE  # odd sections
    assert fc_ex(lib, rope=rope3d(dw=16)) == SHAPE  # sections do not sum to d
    assert fc_ex(lib, rope=rope3d(dt_=-2, dh=42)) == SHAPE
    assert fc_ex(lib, rope=rope3d(theta=0.0)) == VALUE
    assert fc_ex(lib, rope=rope3d(theta=float("nan"))) == VALUE
    assert fc_ex(lib, rope=rope3d(off=1 << 30)) == VALUE
    # the matrix-core table: 1 + 1024 * 12 + 1 * 12 + 8 * 8 entries > 3072
    assert fc_ex(lib, T=1024, rope=rope3d(gh=1024, gw=1)) == UNSUP
    assert "rope table" in lib.gla_last_error().decode()
    # strides
    lay = (N * H * d, d, H * d)
    assert fc_ex(lib, k=tview(FAKE + 0x1000000, lay[0], -d, lay[2])) == SHAPE
    assert fc_ex(lib, v=tview(FAKE + 0x2000000, lay[0], d + 4, lay[2])) == ALIGN  # 8 bytes
    assert fc_ex(lib, g=tview(FAKE + 0x3000008, *lay)) == ALIGN
    # output rows that coincide, or an output reaching into an input
    assert fc_ex(lib, o=tview(FAKE + 0x4000000, lay[0], d, 0)) == ALIAS
    assert "rows overlap" in lib.gla_last_error().decode()
    assert fc_ex(lib, o=tview(FAKE + 0x4000000, lay[0], 0, lay[2])) == ALIAS
    assert fc_ex(lib, o=tview(FAKE + 0x100, *lay)) == ALIAS
    # absent tensors
    assert fc_ex(lib, q=tview(0, *lay)) == NULL
    # empty problems pass validation and launch nothing
    assert fc_ex(lib, B=0) == OK
    # without rotary positions the same checks apply
    assert fc_ex(lib, rope=None, o=tview(FAKE + 0x4000000, lay[0], d, 0)) == ALIAS


def test_ex_workspace(lib):
    r = gla.Rope3D(23, 40, 24, 20, 20, 10000.0)
    # positions need the frame structure: the frame-causal workspace
    assert gla.gla_fwd_bidir_ex_workspace(1, 32, 241, 920, 64, r) == \
        gla.gla_fwd_framecausal_workspace(1, 32, 241, 920, 64)
    # without them the sequence is one frame of F * T tokens
    assert gla.gla_fwd_bidir_ex_workspace(1, 32, 21, 920, 64) == \
        gla.gla_fwd_bidir_workspace(1, 32, 21 * 920, 64)


def test_anchor_validation(lib):
    """gla_softmax_anchor rejects bad arguments before any launch; empty
    problems return OK without touching the device."""
    f = lib.gla_softmax_anchor
    A = FAKE
    B = FAKE + 0x100000  # a second, disjoint aligned address

    def call(q=A, k=B, v=B + 0x100000, g=B + 0x200000, o=B + 0x300000, Bn=1, H=2, Fq=2, F=3,
             T=8, d=64, dt=BF16, causal=1, n_sink=1, window=2, scale=0.125):
        return f(p(q), p(k), p(v), p(g), p(o), Bn, H, Fq, F, T, d, dt, causal, n_sink, window,
                 ctypes.c_float(scale), None)

    assert call(d=48) == UNSUP
    assert call(dt=7) == UNSUP
    assert call(Fq=4) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(causal=2) == VALUE
    assert call(n_sink=-1) == VALUE
    assert call(scale=0.0) == VALUE
    assert call(scale=float("nan")) == VALUE
    assert call(q=0) == NULL
    assert call(o=0) == NULL
    assert call(q=A + 8) == ALIGN
    assert call(o=A) == ALIAS         # o is q
    assert call(o=B + 64) == ALIAS    # o inside k
    # nothing to do: no query tokens, or no heads
    assert call(Fq=0, q=0, g=0, o=0) == OK
    assert call(T=0, q=0, k=0, v=0, g=0, o=0) == OK
    assert call(Bn=0) == OK


def test_states_workspace_sizes(lib):
    # the backward given the states keeps only the adjoint sums: the recomputed
    # slots (one state per slab and frame at 720p/60s) are not needed
    E = 64 * 64 + 64
    full = gla.gla_bwd_framecausal_workspace(1, 32, 241, 920, 64)
    given = gla.gla_bwd_framecausal_states_workspace(1, 32, 241, 920, 64)
    assert full - given == 32 * 241 * E * 4
    assert gla.gla_bwd_framecausal_states_workspace(0, 32, 241, 920, 64) == 0
    assert gla.gla_bwd_framecausal_states_workspace(1, 1, -1, 4, 64) == 0


def test_states_validation(lib):
    """The *_states calls: states required, aligned, and disjoint from the
    other tensors (an output in the forward, an input in the backward)."""
    st = FAKE + 0x9000000
    t = [FAKE + i * 0x1000000 for i in range(9)]  # q k v g o/dO dq dk dv dg
    gam = FAKE + 0xA000000
    dgam = FAKE + 0xB000000
    ws = FAKE + 0xC000000

    def fwd(q=t[0], o=t[4], states=st, B=1, H=1, F=2, T=32, d=64, ws=ws, wsb=1 << 30):
        return lib.gla_fwd_framecausal_states(
            p(q), p(t[1]), p(t[2]), p(t[3]), p(gam), None, None, p(o), None, None, p(states),
            B, H, F, T, d, BF16, ctypes.c_float(1e-6), p(ws), wsb, None)

    def bwd(states=st, dq=t[5], B=1, H=1, F=2, T=32, d=64, ws=ws, wsb=1 << 30):
        return lib.gla_bwd_framecausal_states(
            p(t[0]), p(t[1]), p(t[2]), p(t[3]), p(gam), None, None, p(states), p(t[4]), None,
            None, p(dq), p(t[6]), p(t[7]), p(t[8]), p(dgam), None, None, B, H, F, T, d, BF16,
            ctypes.c_float(1e-6), p(ws), wsb, None)

    assert fwd(states=0) == NULL
    assert "states" in lib.gla_last_error().decode()
    assert fwd(states=st + 8) == ALIGN
    assert fwd(states=t[0] + 256) == ALIAS      # inside q
    assert fwd(states=ws) == ALIAS              # the workspace
    assert fwd(o=st) == ALIAS                   # o over the states
    assert fwd(d=48) == UNSUP
    assert fwd(wsb=0) == WS
    assert fwd(B=0) == OK
    assert bwd(states=0) == NULL
    assert bwd(states=st + 4) == ALIGN
    assert bwd(dq=st) == ALIAS                  # an output over the states
    assert bwd(states=ws) == ALIAS              # the workspace over the states
    assert bwd(wsb=16) == WS
    assert bwd(T=-1) == SHAPE
    assert bwd(B=0) == OK


def test_autograd_functions_refuse_cpu_tensors():
    import torch
    from gated_linear_attention_fwd_amd import autograd as ga
    x = torch.zeros(1, 1, 32, 16, requires_grad=True)
    with pytest.raises(ValueError, match="GPU"):
        ga.gla_bidir(x, x, x, x)
    with pytest.raises(ValueError, match="GPU"):
        ga.gla_framecausal(x, x, x, x, torch.zeros(1, 1, 2))


def test_strided_training_validation(lib):
    """The strided training calls: gradients may not overlap one another, also
    when interleaved in one fused buffer (their spans overlap)."""
    H, N, d = 2, 64, 64
    es = 2
    fused = FAKE + 0x1000000  # a [1, N, 3, H, d] buffer: three interleaved views

    def view(base, off, sb, sh, sn):
        return ctypes.byref(gla._Tensor(base + off * es, sb, sh, sn))

    contig = lambda base: view(base, 0, H * N * d, N * d, d)  # noqa: E731
    inter = lambda i: view(fused, i * H * d, N * 3 * H * d, d, 3 * H * d)  # noqa: E731

    def bwd(dq, dk, states=None, wsb=1 << 30):
        return lib.gla_bwd_framecausal_ex(
            inter(0), inter(1), inter(2), contig(FAKE + 0x2000000), p(FAKE + 0x3000000), None,
            None, p(states), contig(FAKE + 0x4000000), None, None, dq, dk,
            contig(FAKE + 0x5000000), contig(FAKE + 0x6000000), None, None, None, 1, H, 2, N // 2,
            d, BF16, ctypes.c_float(1e-6), None, p(FAKE + 0x8000000), wsb, None)

    # inputs interleaved in one fused buffer are fine (only outputs are checked)
    assert bwd(contig(FAKE + 0x7000000), contig(FAKE + 0x7100000), wsb=0) == WS
    # gradients interleaved in one buffer overlap by span
    g2 = FAKE + 0x9000000
    assert bwd(view(g2, 0, N * 3 * H * d, d, 3 * H * d),
               view(g2, H * d, N * 3 * H * d, d, 3 * H * d)) == ALIAS
    # an output view overlapping itself
    assert bwd(view(FAKE + 0x7000000, 0, 0, 0, d), contig(FAKE + 0x7100000)) == ALIAS
    # a misaligned record
    assert bwd(contig(FAKE + 0x7000000), contig(FAKE + 0x7100000), states=FAKE + 0xA000004) == ALIGN
    f = lib.gla_fwd_framecausal_states_ex
    assert f(inter(0), inter(1), inter(2), contig(FAKE + 0x2000000), p(FAKE + 0x3000000), None,
             None, contig(FAKE + 0x4000000), None, None, None, 1, H, 2, N // 2, d, BF16,
             ctypes.c_float(1e-6), None, p(FAKE + 0x8000000), 1 << 30, None) == NULL


def test_rotary_training_validation(lib):
    """Rotary positions in the training calls: the same checks as the forward
    (grid, sections, the matrix-core table of the states' recompute), before
    any launch; gla_bwd_bidir_ex's workspace follows the frames with them."""
    H, F, T, d = 2, 2, 32, 64
    N = F * T
    lay = (N * H * d, d, H * d)
    t = lambda off: tview(FAKE + off, *lay)  # noqa: E731

    def bwd(rope, T_=T, F_=F):
        return lib.gla_bwd_framecausal_ex(
            t(0), t(0x1000000), t(0x2000000), t(0x3000000), p(FAKE + 0x5000000), None, None,
            None, t(0x4000000), None, None, t(0x6000000), t(0x7000000), t(0x9000000),
            t(0xA000000), None, None, None, 1, H, F_, T_, d, BF16, ctypes.c_float(1e-6), rope,
            p(FAKE + 0xB000000), 1 << 30, None)

    assert bwd(rope3d(gh=3)) == SHAPE
    assert bwd(rope3d(dw=16)) == SHAPE
    assert bwd(rope3d(theta=-1.0)) == VALUE
    assert bwd(rope3d(gh=1024, gw=1), T_=1024) == UNSUP
    assert "rope table" in lib.gla_last_error().decode()

    def bidir_bwd(rope, F_=F, T_=T):
        return lib.gla_bwd_bidir_ex(
            t(0), t(0x1000000), t(0x2000000), t(0x3000000), t(0x4000000), t(0x6000000),
            t(0x7000000), t(0x9000000), t(0xA000000), 1, H, F_, T_, d, BF16,
            ctypes.c_float(1e-6), rope, p(FAKE + 0xB000000), 1 << 30, None)

    assert bidir_bwd(rope3d(gh=3)) == SHAPE
    assert bidir_bwd(rope3d(), F_=-1) == SHAPE
    assert bidir_bwd(rope3d(), F_=0, T_=T) == OK  # no tokens
    r = gla.Rope3D(23, 40, 24, 20, 20, 10000.0)
    assert gla.gla_bwd_bidir_ex_workspace(1, 32, 21, 920, 64, r) == \
        gla.gla_bwd_framecausal_workspace(1, 32, 21, 920, 64)
    assert gla.gla_bwd_bidir_ex_workspace(1, 32, 21, 920, 64) == \
        gla.gla_bwd_bidir_workspace(1, 32, 21 * 920, 64)


def test_bindings_refuse_non_dense_states():
    """The state tensors (S, z, their gradients, gamma and the state record)
    reach the library as bare pointers: the bindings refuse views that are not
    dense or of the wrong shape, also on the strided (_ex) entry points, whose
    token tensors may be any view with a unit feature stride. (CPU tensors: the
    checks run before the device check.)"""
    import torch
    B, H, F, T, d = 2, 2, 2, 32, 16
    x = torch.zeros(B, H, F * T, d)
    gamma = torch.ones(B, H, F)
    S = torch.zeros(B, H, d, d)
    z = torch.zeros(B, H, d)
    buf = torch.zeros(B, H, d, 2 * d)
    S_all = torch.zeros(B, 2 * H, d, d)
    bad_S = {"a column slice": buf[..., :d], "a head slice with B > 1": S_all[:, 1:1 + H],
             "a transposed view": S.transpose(2, 3)}
    for what, S_bad in bad_S.items():
        assert not S_bad.is_contiguous(), what
        for fn in (gla.gla_fwd_framecausal_ex, gla.gla_fwd_framecausal):
            with pytest.raises(ValueError, match="contiguous"):
                fn(x, x, x, x, gamma, S_bad, z)
            with pytest.raises(ValueError, match="contiguous"):
                fn(x, x, x, x, gamma, S, z, S_out=S_bad, z_out=z)
        with pytest.raises(ValueError, match="contiguous"):
            gla.gla_state_carry_ex(x, x, gamma, S_bad, z)
        with pytest.raises(ValueError, match="contiguous"):
            gla.gla_bwd_framecausal_ex(x, x, x, x, gamma, x, S_in=S, z_in=z, dS_out=S_bad,
                                       dz_out=z)
    with pytest.raises(ValueError, match="contiguous"):
        gla.gla_fwd_framecausal_ex(x, x, x, x, gamma, S, torch.zeros(B, H, 2 * d)[..., ::2])
    rec = torch.zeros(B, H, d * d + d, F).transpose(2, 3)  # [B, H, F, d*d + d], not dense
    with pytest.raises(ValueError, match="contiguous"):
        gla.gla_fwd_framecausal_states_ex(x, x, x, x, gamma, states=rec)
    with pytest.raises(ValueError, match="contiguous"):
        gla.gla_bwd_framecausal_ex(x, x, x, x, gamma, x, states=rec)
    with pytest.raises(ValueError, match="contiguous"):
        gla.gla_fwd_framecausal_ex(x, x, x, x, torch.ones(B, H, 2 * F)[..., ::2])
    # shapes: a state for fewer slabs would be read past its end
    with pytest.raises(ValueError, match=r"S_in must be float32 \[2, 2, 16, 16\]"):
        gla.gla_fwd_framecausal_ex(x, x, x, x, gamma, S[:1], z[:1])
    with pytest.raises(ValueError, match="z_out must be float32"):
        gla.gla_fwd_framecausal(x, x, x, x, gamma, S_out=S, z_out=torch.zeros(B, H, d + 1))
    with pytest.raises(ValueError, match="dS_out must be float32"):
        gla.gla_bwd_framecausal(x, x, x, x, gamma, x, dS_out=S.double(), dz_out=z)
    with pytest.raises(ValueError, match="S_in must be float32"):
        gla.gla_gdn_framecausal(x, x, x, torch.zeros(B, H, F * T), gamma, S_in=S[:, :1])
    # outputs of the contiguous calls must match the inputs' shape
    with pytest.raises(ValueError, match="out must match"):
        gla.gla_fwd_framecausal(x, x, x, x, gamma, out=torch.zeros(B, H, F * T - 1, d))
    with pytest.raises(ValueError, match="out must match"):
        gla.gla_fwd_bidir(x, x, x, x, out=torch.zeros(B, H, F * T, d, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dq must match"):
        gla.gla_bwd_bidir(x, x, x, x, x, out={"dq": torch.zeros(B, H, 1, d)})
    # the token views themselves may be strided: only their feature axis counts
    xt = torch.zeros(B, F * T, H, d).transpose(1, 2)
    with pytest.raises(ValueError, match="GPU"):
        gla.gla_fwd_framecausal_ex(xt, xt, xt, xt, gamma, S, z)
    with pytest.raises(ValueError, match="unit stride"):
        gla.gla_fwd_framecausal_ex(torch.zeros(B, H, d, F * T).transpose(2, 3), x, x, x, gamma)


def test_rope_table_size_overflow(lib):
    """A latent grid so large that the rotary table's entry count overflows
    32-bit arithmetic is refused before any launch (the count is formed in
    64 bits)."""
    T = 1 << 26
    r = rope3d(gh=T, gw=1, dt_=0, dh=128, dw=0)  # grid_h * dim_h / 2 = 2^32 entries
    assert fc_ex(lib, T=T, F=1, H=1, d=128, rope=r) == SHAPE
    assert "rope" in lib.gla_last_error().decode()


def test_noalloc_refuses_sizes_beyond_its_scratch(lib):
    """gla_fwd_framecausal_noalloc checks the workspace its sizes need against
    the static scratch before any HIP call (so this runs without a GPU)."""
    assert gla.NOALLOC_SCRATCH_BYTES == 256 << 20
    # 720p/60s at H = 32, d = 64 fits; four times the heads does not
    assert gla.gla_fwd_framecausal_workspace(1, 32, 241, 920, 64) <= gla.NOALLOC_SCRATCH_BYTES
    assert gla.gla_fwd_framecausal_workspace(2, 40, 31, 920, 128) <= gla.NOALLOC_SCRATCH_BYTES
    assert gla.gla_fwd_framecausal_workspace(1, 128, 241, 920, 64) > gla.NOALLOC_SCRATCH_BYTES
    f = lib.gla_fwd_framecausal_noalloc
    st = f(p(FAKE), p(FAKE), p(FAKE), p(FAKE), p(FAKE), None, None, p(FAKE + 0x100000), None,
           None, 1, 128, 241, 920, 64, BF16, ctypes.c_float(1e-6), None)
    assert st == WS
    assert "static scratch" in lib.gla_last_error().decode()


def test_stream_probe_validation(lib):
    """The bandwidth probe refuses bad kinds, sizes, pointers and overlaps on
    the host (no launch)."""
    f = lib.gla_stream_probe
    MiB = 1 << 20
    a, b, o = FAKE, FAKE + 0x10000000, FAKE + 0x20000000
    assert f(9, p(a), p(b), p(o), MiB, None) == VALUE
    assert f(-1, p(a), p(b), p(o), MiB, None) == VALUE
    assert f(0, p(a), None, p(o), MiB + 16, None) == SHAPE  # not a multiple of 256 KiB
    assert f(0, p(a), None, p(o), 0, None) == SHAPE
    assert f(0, None, None, p(o), MiB, None) == NULL        # read needs a
    assert f(6, p(a), None, p(o), MiB, None) == NULL        # two reads need b
    assert f(8, p(a), None, p(o), MiB, None) == NULL
    assert f(2, None, None, None, MiB, None) == NULL        # every kind needs out
    assert f(4, p(a + 4), None, p(o), MiB, None) == ALIGN
    assert f(4, p(a), None, p(a + MiB // 2), MiB, None) == ALIAS
