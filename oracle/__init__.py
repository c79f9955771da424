"""fp64 CPU oracle for the gated linear-attention forward pass.

TEST INFRASTRUCTURE ONLY: the plain, slow checker that the GPU library is
compared against. Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the GPU library never does, and this package imports
nothing from it. The arithmetic lives in ``gla_oracle.c`` (plain C, fp64,
OpenMP over independent slabs); this module only builds that file with gcc and
marshals numpy arrays into it.

Formulations (each function returns ``(o, S_out, z_out)`` as float64 arrays):

* :func:`recurrent` -- decay, rank-1 update per token, then the frame readout.
* :func:`quadratic` -- explicit weighted sum over key tokens (O(N^2 d)).
* :func:`chunked`   -- chunk sums of phi(k) v^T, per-frame sum, scan, readout.

Also :func:`backward` (gradients of the same forward), :func:`gdn` (the
frame-wise Gated DeltaNet) and :func:`softmax_anchor` (gated softmax attention
over whole frames with sink frames and a local window).

Definitions followed: the gated linear attention token mixer of "SANA-Video
2.0: Hybrid Linear Attention with Attention Residuals for Efficient Video
Generation" (section "Hybrid Linear-Softmax Attention"), its fixed D x D state
updated additively block by block ("SANA-Video: Efficient Video Generation with
Block Linear Diffusion Transformer", ICLR 2026 oral talk, block KV cache
passage) and frame-wise decay gates ("SANA-WM" analysis page, method
components). The readings where the pages are silent are stated in
``gla_oracle.c``.

Input arrays are ``[B, H, N, d]``; their dtype selects the exact upcast:
``uint16`` holds bfloat16 bit patterns, ``float32`` and ``float64`` are used
as they are. ``gamma`` is ``[B, H, F]``, ``S_in`` ``[B, H, d, d]``, ``z_in``
``[B, H, d]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BIDIR = 0
FRAMECAUSAL = 1


class Rope(ctypes.Structure):
    """3D rotary positions: token l of frame f sits at (frame_offset + f,
    l // grid_w, l % grid_w); pairs of features turn with t, y, x in sections of
    dim_t, dim_h, dim_w features; pair j of an m-pair section by pos * theta**(-j/m)."""
    _fields_ = [("grid_h", ctypes.c_int), ("grid_w", ctypes.c_int),
                ("frame_offset", ctypes.c_int), ("dim_t", ctypes.c_int),
                ("dim_h", ctypes.c_int), ("dim_w", ctypes.c_int), ("theta", ctypes.c_double)]

_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def build(force: bool = True) -> str:
    """Compile ``gla_oracle.c`` into ``liboracle.so`` next to it (gcc, fp64)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    common = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
              ctypes.c_double]
    lib.gla_oracle_recurrent.argtypes = common + [ctypes.c_int]
    lib.gla_oracle_quadratic.argtypes = common + [ctypes.c_int]
    lib.gla_oracle_chunked.argtypes = common + [ctypes.c_int, ctypes.c_int]
    for fn in (lib.gla_oracle_recurrent, lib.gla_oracle_quadratic, lib.gla_oracle_chunked):
        fn.restype = ctypes.c_int
    lib.gla_oracle_max_threads.restype = ctypes.c_int
    lib.gla_oracle_rope_recurrent.argtypes = common + [ctypes.POINTER(Rope), ctypes.c_int]
    lib.gla_oracle_rope_recurrent.restype = ctypes.c_int
    lib.gla_oracle_rope_quadratic.argtypes = common[:10] + common[12:] + [
        ctypes.POINTER(Rope), ctypes.c_int]
    lib.gla_oracle_rope_quadratic.restype = ctypes.c_int
    lib.gla_oracle_backward.argtypes = [ctypes.c_int, ctypes.c_int] + [vp] * 17 + [
        ctypes.c_int] * 5 + [ctypes.c_double, ctypes.POINTER(Rope), ctypes.c_int, ctypes.c_int]
    lib.gla_oracle_backward.restype = ctypes.c_int
    lib.gla_oracle_gdn.argtypes = [ctypes.c_int] + [vp] * 8 + [ctypes.c_int] * 5 + [
        ctypes.c_double, ctypes.c_int]
    lib.gla_oracle_gdn.restype = ctypes.c_int
    lib.gla_oracle_softmax_anchor.argtypes = [ctypes.c_int] + [vp] * 5 + [ctypes.c_int] * 9 + [
        ctypes.c_double, ctypes.c_int]
    lib.gla_oracle_softmax_anchor.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    """Threads the oracle's OpenMP runtime would use by default."""
    return int(_load().gla_oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(mode, q, k, v, g, gamma, S_in, z_in, F, T, outputs):
    k = np.ascontiguousarray(k)
    if k.ndim != 4:
        raise ValueError("k must be [B, H, N, d]")
    B, H, N, d = k.shape
    dt = _DT.get(k.dtype)
    if dt is None:
        raise TypeError("unsupported input dtype %s" % k.dtype)
    v = np.ascontiguousarray(v)
    arrays = [v]
    if outputs:
        q = np.ascontiguousarray(q)
        g = np.ascontiguousarray(g)
        arrays += [q, g]
    else:
        q = g = None
    for a in arrays:
        if a.shape != k.shape or a.dtype != k.dtype:
            raise ValueError("q, k, v, g must share shape and dtype")
    if mode == BIDIR:
        F, T = 1, N
        gamma = S_in = z_in = None
    else:
        if F is None:
            if gamma is None:
                raise ValueError("frame-causal mode needs F (or gamma)")
            F = np.shape(gamma)[-1]
        if T is None:
            T = N // F
        if F * T != N:
            raise ValueError("N must equal F * T")
        gamma = np.ascontiguousarray(np.broadcast_to(np.asarray(gamma, np.float64), (B, H, F)))
        if S_in is not None:
            S_in = np.ascontiguousarray(np.asarray(S_in, np.float64).reshape(B, H, d, d))
        if z_in is not None:
            z_in = np.ascontiguousarray(np.asarray(z_in, np.float64).reshape(B, H, d))
    o = np.empty((B, H, N, d), np.float64) if outputs else None
    S_out = np.empty((B, H, d, d), np.float64)
    z_out = np.empty((B, H, d), np.float64)
    return q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d, dt


def _run(fn, mode, q, k, v, g, gamma, S_in, z_in, F, T, eps, outputs, extra, nthreads):
    (q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d, dt) = _prep(
        mode, q, k, v, g, gamma, S_in, z_in, F, T, outputs)
    fn(mode, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in),
       _ptr(o), _ptr(S_out), _ptr(z_out), B, H, F, T, d, float(eps), *extra, int(nthreads))
    return o, S_out, z_out


def recurrent(mode, q, k, v, g, gamma=None, S_in=None, z_in=None, F=None, T=None,
              eps=1e-6, outputs=True, nthreads=0):
    """Recurrent form R. ``outputs=False`` computes only (S_out, z_out)."""
    return _run(_load().gla_oracle_recurrent, mode, q, k, v, g, gamma, S_in, z_in, F, T, eps,
                outputs, (), nthreads)


def quadratic(mode, q, k, v, g, gamma=None, S_in=None, z_in=None, F=None, T=None,
              eps=1e-6, outputs=True, nthreads=0):
    """Quadratic brute-force form Q (O(N^2 d) per slab: small inputs only)."""
    return _run(_load().gla_oracle_quadratic, mode, q, k, v, g, gamma, S_in, z_in, F, T, eps,
                outputs, (), nthreads)


def chunked(mode, q, k, v, g, gamma=None, S_in=None, z_in=None, F=None, T=None,
            eps=1e-6, C=7, outputs=True, nthreads=0):
    """Chunked form C with chunk length ``C`` (the last chunk of a frame may be shorter)."""
    return _run(_load().gla_oracle_chunked, mode, q, k, v, g, gamma, S_in, z_in, F, T, eps,
                outputs, (int(C),), nthreads)


def _rope(rope, T, d):
    r = rope if isinstance(rope, Rope) else Rope(**rope)
    if r.grid_h * r.grid_w != T or r.dim_t + r.dim_h + r.dim_w != d:
        raise ValueError("rope grid must cover T tokens and its sections d features")
    if any(x % 2 for x in (r.dim_t, r.dim_h, r.dim_w)):
        raise ValueError("rope sections must be even")
    return r


def rope_recurrent(mode, q, k, v, g, gamma=None, S_in=None, z_in=None, F=None, T=None,
                   eps=1e-6, rope=None, outputs=True, nthreads=0):
    """Recurrent form with 3D rotary positions (numerator rotated, normaliser not).

    In bidirectional mode F and T give the positions (N = F * T)."""
    lib = _load()
    if mode == BIDIR:
        N = np.shape(k)[2]
        Fp, Tp = (F, T) if F else (1, N)
        q_, k_, v_, g_, _, _, _, o, S_out, z_out, B, H, _, _, d, dt = _prep(
            BIDIR, q, k, v, g, None, None, None, None, None, outputs)
        r = _rope(rope, Tp, d)
        lib.gla_oracle_rope_recurrent(BIDIR, dt, _ptr(q_), _ptr(k_), _ptr(v_), _ptr(g_), None,
                                      None, None, _ptr(o), _ptr(S_out), _ptr(z_out), B, H, Fp, Tp,
                                      d, float(eps), ctypes.byref(r), int(nthreads))
        return o, S_out, z_out
    (q_, k_, v_, g_, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d, dt) = _prep(
        mode, q, k, v, g, gamma, S_in, z_in, F, T, outputs)
    r = _rope(rope, T, d)
    lib.gla_oracle_rope_recurrent(mode, dt, _ptr(q_), _ptr(k_), _ptr(v_), _ptr(g_), _ptr(gamma),
                                  _ptr(S_in), _ptr(z_in), _ptr(o), _ptr(S_out), _ptr(z_out), B, H,
                                  F, T, d, float(eps), ctypes.byref(r), int(nthreads))
    return o, S_out, z_out


def rope_quadratic(mode, q, k, v, g, gamma=None, S_in=None, z_in=None, F=None, T=None,
                   eps=1e-6, rope=None, nthreads=0):
    """Quadratic form with 3D rotary positions; returns o only."""
    lib = _load()
    if mode == BIDIR:
        N = np.shape(k)[2]
        Fp, Tp = (F, T) if F else (1, N)
        q_, k_, v_, g_, _, _, _, o, _, _, B, H, _, _, d, dt = _prep(
            BIDIR, q, k, v, g, None, None, None, None, None, True)
        r = _rope(rope, Tp, d)
        lib.gla_oracle_rope_quadratic(BIDIR, dt, _ptr(q_), _ptr(k_), _ptr(v_), _ptr(g_), None,
                                      None, None, _ptr(o), B, H, Fp, Tp, d, float(eps),
                                      ctypes.byref(r), int(nthreads))
        return o
    (q_, k_, v_, g_, gamma, S_in, z_in, o, _, _, B, H, F, T, d, dt) = _prep(
        mode, q, k, v, g, gamma, S_in, z_in, F, T, True)
    r = _rope(rope, T, d)
    lib.gla_oracle_rope_quadratic(mode, dt, _ptr(q_), _ptr(k_), _ptr(v_), _ptr(g_), _ptr(gamma),
                                  _ptr(S_in), _ptr(z_in), _ptr(o), B, H, F, T, d, float(eps),
                                  ctypes.byref(r), int(nthreads))
    return o


def backward(mode, q, k, v, g, dO, gamma=None, S_in=None, z_in=None, dS_out=None,
             dz_out=None, F=None, T=None, eps=1e-6, rope=None, nthreads=0):
    """Gradients of the forward definition (chain rule, fp64) for
    dL/do = dO and, in frame-causal mode, dL/dS_out = dS_out, dL/dz_out = dz_out.

    With ``rope`` the gradients are those of the rotary form
    (:func:`rope_recurrent`); in bidirectional mode F and T then give the
    positions (N = F * T), as there.

    Returns a dict with dq, dk, dv, dg ([B, H, N, d] float64) and, in
    frame-causal mode, dgamma [B, H, F], dS_in [B, H, d, d], dz_in [B, H, d]."""
    pos_T = None
    if rope is not None and mode == BIDIR:
        pos_T = T if F else np.shape(k)[2]
        F = T = None
    (q, k, v, g, gamma, S_in, z_in, _, _, _, B, H, F, T, d, dt) = _prep(
        mode, q, k, v, g, gamma, S_in, z_in, F, T, True)
    r = None
    if rope is not None:
        pos_T = T if pos_T is None else pos_T
        r = _rope(rope, pos_T, d)
        if (F * T) % pos_T:
            raise ValueError("the positions need whole frames of grid_h * grid_w tokens")
    dO = np.ascontiguousarray(bf16_to_f64(dO) if np.asarray(dO).dtype == np.uint16
                              else np.asarray(dO, np.float64))
    if dO.shape != (B, H, F * T, d):
        raise ValueError("dO must be [B, H, N, d]")
    causal = mode == FRAMECAUSAL
    if causal and dS_out is not None:
        dS_out = np.ascontiguousarray(np.asarray(dS_out, np.float64).reshape(B, H, d, d))
    else:
        dS_out = None
    if causal and dz_out is not None:
        dz_out = np.ascontiguousarray(np.asarray(dz_out, np.float64).reshape(B, H, d))
    else:
        dz_out = None
    shape = (B, H, F * T, d)
    out = {n: np.empty(shape, np.float64) for n in ("dq", "dk", "dv", "dg")}
    if causal:
        out["dgamma"] = np.empty((B, H, F), np.float64)
        out["dS_in"] = np.empty((B, H, d, d), np.float64)
        out["dz_in"] = np.empty((B, H, d), np.float64)
    _load().gla_oracle_backward(
        mode, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in),
        _ptr(dO), _ptr(dS_out), _ptr(dz_out), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out.get("dgamma")), _ptr(out.get("dS_in")),
        _ptr(out.get("dz_in")), B, H, F, T, d, float(eps),
        ctypes.byref(r) if r is not None else None, int(pos_T or T), int(nthreads))
    return out


def gdn(q, k, v, beta, gamma, S_in=None, key_scale=None, T=None, outputs=True, nthreads=0):
    """Frame-wise Gated DeltaNet (block delta rule per frame); returns (o, S_out).

    q, k, v [B, H, N, d]; beta [B, H, N] (write strengths); gamma [B, H, F]
    (frame decays, F = gamma.shape[-1], T = N / F); key_scale defaults to
    1 / sqrt(d T)."""
    k = np.ascontiguousarray(k)
    B, H, N, d = k.shape
    dt = _DT.get(k.dtype)
    if dt is None:
        raise TypeError("unsupported input dtype %s" % k.dtype)
    v = np.ascontiguousarray(v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must share shape and dtype")
    if outputs:
        q = np.ascontiguousarray(q)
        if q.shape != k.shape or q.dtype != k.dtype:
            raise ValueError("q must match k")
    else:
        q = None
    gamma = np.ascontiguousarray(np.asarray(gamma, np.float64))
    F = gamma.shape[-1]
    T = N // F if T is None else T
    if F * T != N or gamma.shape != (B, H, F):
        raise ValueError("gamma must be [B, H, F] with N = F * T")
    beta = np.ascontiguousarray(np.broadcast_to(np.asarray(beta, np.float64), (B, H, N)))
    if S_in is not None:
        S_in = np.ascontiguousarray(np.asarray(S_in, np.float64).reshape(B, H, d, d))
    if key_scale is None:
        key_scale = 1.0 / np.sqrt(d * T)
    o = np.empty((B, H, N, d), np.float64) if outputs else None
    S_out = np.empty((B, H, d, d), np.float64)
    _load().gla_oracle_gdn(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma), _ptr(S_in),
                           _ptr(o), _ptr(S_out), B, H, F, T, d, float(key_scale), int(nthreads))
    return o, S_out


def softmax_anchor(q, k, v, g, T, causal=True, n_sink=0, window=0, scale=None, nthreads=0):
    """Gated softmax attention over whole frames; returns o (float64, shaped like q).

    k, v [B, H, F*T, d] (F key frames of T tokens); q, g [B, H, Fq*T, d], the
    tokens of the last Fq key frames. Full mode (causal False): every key is
    visible. Frame-causal: query frame f sees key frames i <= f with
    i < n_sink (sinks) or i > f - window (window <= 0: no limit). scale
    defaults to 1/sqrt(d)."""
    k = np.ascontiguousarray(k)
    B, H, Nk, d = k.shape
    dt = _DT.get(k.dtype)
    if dt is None:
        raise TypeError("unsupported input dtype %s" % k.dtype)
    v = np.ascontiguousarray(v)
    q = np.ascontiguousarray(q)
    g = np.ascontiguousarray(g)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must share shape and dtype")
    if q.shape[:2] != (B, H) or q.shape[3] != d or q.dtype != k.dtype or g.shape != q.shape \
            or g.dtype != q.dtype:
        raise ValueError("q and g must be [B, H, Nq, d] in k's dtype")
    Nq = q.shape[2]
    if T <= 0 or Nk % T or Nq % T or Nq > Nk:
        raise ValueError("Nq and Nk must be multiples of T with Nq <= Nk")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, Nq, d), np.float64)
    _load().gla_oracle_softmax_anchor(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), B, H,
                                      Nq // T, Nk // T, T, d, int(bool(causal)), int(n_sink),
                                      int(window), float(scale), int(nthreads))
    return o


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


if __name__ == "__main__":  # pragma: no cover
    print(build())
    sys.exit(0)
