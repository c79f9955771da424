"""MI355X-native gated linear-attention forward pass.

A thin Python binding over ``libgla.so``, the C-ABI library whose entry points
are declared in ``include/gla.h``. Every step of the computation runs in that
library's HIP kernels; this module only checks and marshals arguments, and uses
PyTorch for device memory and streams. If the library is not built, every call
raises: there is no CPU fallback.

Entry points (same names as the C ABI):

* :func:`gla_fwd_bidir` -- bidirectional (whole-sequence) gated linear attention
* :func:`gla_fwd_framecausal` -- frame-causal attention with per-frame decay and
  an optional carried state (the block KV cache)
* :func:`gla_state_carry` -- the carried state after more frames, from k, v only
* :func:`gla_fwd_bidir_ex`, :func:`gla_fwd_framecausal_ex`,
  :func:`gla_state_carry_ex` -- the same on any [B, H, N, d]-shaped view whose
  feature axis is contiguous (e.g. ``x.transpose(1, 2)`` of a [B, N, H, d]
  tensor, or slices of a fused [B, N, 3, H, d] projection), with optional 3D
  rotary positions (:class:`Rope3D`)
* :func:`gla_bwd_framecausal`, :func:`gla_bwd_bidir` -- the backward pass
  (dq, dk, dv, dg, dgamma and the carried-state gradients)
* :func:`gla_fwd_framecausal_states`, :func:`gla_bwd_framecausal_states` -- the
  forward keeping every frame's state and the backward that reads it
* :mod:`.autograd` -- the two modes as ``torch.autograd`` functions (forward and
  backward both through the calls above)
* :func:`gla_gdn_framecausal` -- the frame-wise Gated DeltaNet mixer (a block
  delta-rule update per frame, keys scaled by 1/sqrt(d T))
* ``gla_*_workspace`` -- workspace sizes in bytes

The operation is the gated linear attention token mixer of "SANA-Video 2.0:
Hybrid Linear Attention with Attention Residuals for Efficient Video
Generation" (section "Hybrid Linear-Softmax Attention"), with the fixed D x D
state and additive per-block update of the SANA-Video ICLR 2026 oral talk
(block KV cache passage) and frame-wise decay gates ("SANA-WM" analysis page).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "GlaError", "Rope3D", "gla_fwd_bidir", "gla_fwd_framecausal", "gla_state_carry",
    "gla_fwd_bidir_ex", "gla_fwd_framecausal_ex", "gla_state_carry_ex",
    "gla_fwd_bidir_workspace", "gla_fwd_framecausal_workspace", "gla_state_carry_workspace",
    "gla_fwd_bidir_ex_workspace", "gla_bwd_framecausal", "gla_bwd_bidir",
    "gla_bwd_framecausal_workspace", "gla_bwd_bidir_workspace", "gla_fwd_framecausal_states",
    "gla_bwd_framecausal_states", "gla_bwd_framecausal_states_workspace",
    "gla_fwd_framecausal_states_ex", "gla_bwd_framecausal_ex", "gla_bwd_bidir_ex",
    "gla_bwd_bidir_ex_workspace", "gla_gdn_framecausal",
    "gla_gdn_framecausal_workspace", "gla_softmax_anchor", "gla_fwd_framecausal_noalloc",
    "NOALLOC_SCRATCH_BYTES", "library_path", "load_library",
    "profile_begin", "profile_end", "stream_probe", "PROBE_KINDS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgla.so")
_lib = None

GLA_F32 = 0
GLA_BF16 = 1
# the static device scratch of gla_fwd_framecausal_noalloc (GLA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20


class GlaError(RuntimeError):
    """A non-OK status from libgla (the message carries the library's detail)."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__("libgla status %d (%s): %s" % (status, name, detail))
        self.status = status


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 16), ("launches", ctypes.c_int),
                ("total_ms", ctypes.c_double)]


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class Rope3D(ctypes.Structure):
    """3D rotary positions (``gla_rope3d``): token l of frame f sits at
    (frame_offset + f, l // grid_w, l % grid_w); feature pairs form sections of
    dim_t, dim_h and dim_w features turning with each axis, pair j of an m-pair
    section by pos * theta ** (-j / m)."""
    _fields_ = [("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("frame_offset", ctypes.c_int32), ("dim_t", ctypes.c_int32),
                ("dim_h", ctypes.c_int32), ("dim_w", ctypes.c_int32),
                ("theta", ctypes.c_double)]

    def __init__(self, grid_h: int, grid_w: int, dim_t: int, dim_h: int, dim_w: int,
                 theta: float = 10000.0, frame_offset: int = 0):
        super().__init__(grid_h, grid_w, frame_offset, dim_t, dim_h, dim_w, theta)

    @classmethod
    def video(cls, grid_h: int, grid_w: int, d: int, theta: float = 10000.0,
              frame_offset: int = 0) -> "Rope3D":
        """The common video split of a head: 2 * (d // 6) features each for the
        row and column axes, the rest (a multiple of 4) for the frame axis."""
        s = 2 * (d // 6)
        return cls(grid_h, grid_w, d - 2 * s, s, s, theta, frame_offset)

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgla.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libgla.so is not built (%s); run `python -m "
                           "gated_linear_attention_fwd_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.gla_fwd_bidir_workspace.argtypes = [i32, i32, i64, i32]
    lib.gla_fwd_bidir_workspace.restype = sz
    lib.gla_fwd_framecausal_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.gla_fwd_framecausal_workspace.restype = sz
    lib.gla_state_carry_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.gla_state_carry_workspace.restype = sz
    lib.gla_fwd_bidir.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, f32, vp, sz, vp]
    lib.gla_fwd_bidir.restype = i32
    lib.gla_fwd_framecausal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                        i32, i32, i32, f32, vp, sz, vp]
    lib.gla_fwd_framecausal.restype = i32
    lib.gla_state_carry.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                    sz, vp]
    lib.gla_state_carry.restype = i32
    lib.gla_fwd_framecausal_noalloc.argtypes = [vp] * 10 + [i32] * 6 + [f32, vp]
    lib.gla_fwd_framecausal_noalloc.restype = i32
    tp, rp = ctypes.POINTER(_Tensor), ctypes.POINTER(Rope3D)
    lib.gla_fwd_bidir_ex_workspace.argtypes = [i32, i32, i32, i32, i32, rp]
    lib.gla_fwd_bidir_ex_workspace.restype = sz
    lib.gla_fwd_bidir_ex.argtypes = [tp, tp, tp, tp, tp, i32, i32, i32, i32, i32, i32, f32, rp,
                                     vp, sz, vp]
    lib.gla_fwd_bidir_ex.restype = i32
    lib.gla_fwd_framecausal_ex.argtypes = [tp, tp, tp, tp, vp, vp, vp, tp, vp, vp, i32, i32, i32,
                                           i32, i32, i32, f32, rp, vp, sz, vp]
    lib.gla_fwd_framecausal_ex.restype = i32
    lib.gla_state_carry_ex.argtypes = [tp, tp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                       rp, vp, sz, vp]
    lib.gla_state_carry_ex.restype = i32
    lib.gla_bwd_framecausal_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.gla_bwd_framecausal_workspace.restype = sz
    lib.gla_bwd_bidir_workspace.argtypes = [i32, i32, i64, i32]
    lib.gla_bwd_bidir_workspace.restype = sz
    lib.gla_bwd_framecausal.argtypes = [vp] * 17 + [i32] * 6 + [f32, vp, sz, vp]
    lib.gla_bwd_framecausal.restype = i32
    lib.gla_bwd_bidir.argtypes = [vp] * 9 + [i32, i32, i64, i32, i32, f32, vp, sz, vp]
    lib.gla_bwd_bidir.restype = i32
    lib.gla_fwd_framecausal_states.argtypes = [vp] * 11 + [i32] * 6 + [f32, vp, sz, vp]
    lib.gla_fwd_framecausal_states.restype = i32
    lib.gla_bwd_framecausal_states_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.gla_bwd_framecausal_states_workspace.restype = sz
    lib.gla_bwd_framecausal_states.argtypes = [vp] * 18 + [i32] * 6 + [f32, vp, sz, vp]
    lib.gla_bwd_framecausal_states.restype = i32
    lib.gla_fwd_framecausal_states_ex.argtypes = [tp, tp, tp, tp, vp, vp, vp, tp, vp, vp, vp] + \
        [i32] * 6 + [f32, rp, vp, sz, vp]
    lib.gla_fwd_framecausal_states_ex.restype = i32
    lib.gla_bwd_framecausal_ex.argtypes = [tp, tp, tp, tp, vp, vp, vp, vp, tp, vp, vp, tp, tp, tp,
                                           tp, vp, vp, vp] + [i32] * 6 + [f32, rp, vp, sz, vp]
    lib.gla_bwd_framecausal_ex.restype = i32
    lib.gla_bwd_bidir_ex_workspace.argtypes = [i32, i32, i32, i32, i32, rp]
    lib.gla_bwd_bidir_ex_workspace.restype = sz
    lib.gla_bwd_bidir_ex.argtypes = [tp] * 9 + [i32] * 6 + [f32, rp, vp, sz, vp]
    lib.gla_bwd_bidir_ex.restype = i32
    lib.gla_gdn_framecausal_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.gla_gdn_framecausal_workspace.restype = sz
    lib.gla_gdn_framecausal.argtypes = [vp] * 8 + [i32] * 6 + [f32, vp, sz, vp]
    lib.gla_gdn_framecausal.restype = i32
    lib.gla_softmax_anchor.argtypes = [vp] * 5 + [i32] * 10 + [f32, vp]
    lib.gla_softmax_anchor.restype = i32
    lib.gla_status_string.argtypes = [i32]
    lib.gla_status_string.restype = ctypes.c_char_p
    lib.gla_last_error.argtypes = []
    lib.gla_last_error.restype = ctypes.c_char_p
    lib.gla_version.restype = i32
    lib.gla_stream_probe.argtypes = [i32, vp, vp, vp, sz, vp]
    lib.gla_stream_probe.restype = i32
    lib.gla_profile_begin.argtypes = [i32]
    lib.gla_profile_begin.restype = i32
    lib.gla_profile_end.argtypes = [ctypes.POINTER(_KernelTime), i32, ctypes.POINTER(i32)]
    lib.gla_profile_end.restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise GlaError(status, lib.gla_status_string(status).decode(),
                       lib.gla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GLA_F32
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    raise TypeError("inputs must be float32 or bfloat16, got %s" % t.dtype)


def _require_device(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libgla runs on the GPU only; got a tensor on %s" % t.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _require_device_any_layout(*views: Optional[torch.Tensor],
                               dense=()) -> torch.device:
    """Like _require_device, for the strided entry points: the token tensors
    (``views``, [B, H, N, d]) may have any layout whose last (feature) axis has
    unit stride; every other tensor (``dense``: gamma, states, the state
    record, fp32 gradients, the workspace) reaches the library as a bare
    pointer and must be contiguous."""
    dev = None
    for t in views:
        if t is None:
            continue
        if t.dim() != 4:
            raise ValueError("token tensors must be [B, H, N, d] views")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("the feature axis must have unit stride")
    for t in dense:
        if t is not None and not t.is_contiguous():
            raise ValueError("gamma, the states, the state record, the fp32 gradients and the "
                             "workspace must be contiguous")
    for t in (*views, *dense):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libgla runs on the GPU only; got a tensor on %s" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _dense(t: Optional[torch.Tensor], shape, name: str) -> None:
    """A float32 tensor the library reads or writes through a bare pointer
    (states, normalisers, their gradients): exact shape, dense layout."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32:
        raise ValueError("%s must be float32 %s, got %s %s"
                         % (name, list(shape), t.dtype, list(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _states(B: int, H: int, d: int, **ts: Optional[torch.Tensor]) -> None:
    """_dense for S-like ([B, H, d, d]: names starting with S or dS) and
    z-like ([B, H, d]) tensors."""
    for name, t in ts.items():
        square = name.startswith("S") or name.startswith("dS")
        _dense(t, (B, H, d, d) if square else (B, H, d), name)


def _like(t: torch.Tensor, ref: torch.Tensor, name: str) -> None:
    if t.shape != ref.shape or t.dtype != ref.dtype:
        raise ValueError("%s must match q's shape and dtype" % name)


def _view(t: Optional[torch.Tensor]):
    """gla_tensor of a [B, H, N, d] view (NULL data when absent or empty)."""
    if t is None:
        return None
    sb, sh, sn, _ = t.stride()
    return ctypes.byref(_Tensor(t.data_ptr() if t.numel() else None, sb, sh, sn))


def _rope(rope):
    if rope is None:
        return None
    r = rope if isinstance(rope, Rope3D) else Rope3D(**rope)
    return ctypes.byref(r)


def _qkvg(*ts: Optional[torch.Tensor]):
    ref = next(t for t in ts if t is not None)
    if ref.dim() != 4:
        raise ValueError("q, k, v, g must be [B, H, N, d]")
    for t in ts:
        if t is not None and (t.shape != ref.shape or t.dtype != ref.dtype):
            raise ValueError("q, k, v, g must share shape and dtype")
    return ref


def _stream_handle(stream, device, *tensors):
    """The raw stream the kernels are launched on (the current stream if None).

    When it is another stream, every tensor of the call (inputs, outputs and
    the workspace, which the binding may have allocated on the current stream)
    is recorded as in use by it, so that torch's caching allocator does not
    hand their memory out again while the kernels still run there."""
    current = torch.cuda.current_stream(device)
    if stream is None:
        stream = current
    elif not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    if stream != current:
        for t in tensors:
            for x in (t.values() if isinstance(t, dict) else (t,)):
                if isinstance(x, torch.Tensor) and x.is_cuda and x.numel():
                    x.record_stream(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def gla_fwd_bidir_workspace(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().gla_fwd_bidir_workspace(B, H, N, d))


def gla_fwd_framecausal_workspace(B: int, H: int, F: int, T: int, d: int) -> int:
    return int(load_library().gla_fwd_framecausal_workspace(B, H, F, T, d))


def gla_state_carry_workspace(B: int, H: int, F: int, T: int, d: int) -> int:
    return int(load_library().gla_state_carry_workspace(B, H, F, T, d))


def gla_fwd_bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  eps: float = 1e-6, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """o = sigmoid(g) * phi(q) S / (phi(q) z + eps) with one state over all N tokens."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    o = torch.empty_like(ref) if out is None else out
    _like(o, ref, "out")
    dev = _require_device(q, k, v, g, o, workspace)
    B, H, N, d = ref.shape
    ws, wsb = _workspace(lib.gla_fwd_bidir_workspace(B, H, N, d), dev, workspace)
    _check(lib.gla_fwd_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), B, H, N, d,
                             dt, eps, _ptr(ws), wsb,
                             _stream_handle(stream, dev, q, k, v, g, o, ws)))
    return o


def gla_fwd_framecausal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        gamma: torch.Tensor, S_in: Optional[torch.Tensor] = None,
                        z_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                        out: Optional[torch.Tensor] = None, S_out: Optional[torch.Tensor] = None,
                        z_out: Optional[torch.Tensor] = None, return_state: bool = False,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """Frame-causal gated linear attention; F = gamma.shape[-1], T = N / F.

    Returns ``o``, or ``(o, S_out, z_out)`` when ``return_state`` is set or
    S_out/z_out are given (S_out may be S_in for an in-place carry)."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if F == 0 or N % F:
        if not (F == 0 and N == 0):
            raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    want_state = return_state or S_out is not None or z_out is not None
    if want_state and S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if want_state and z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    o = torch.empty_like(ref) if out is None else out
    _like(o, ref, "out")
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device(q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, workspace)
    ws, wsb = _workspace(lib.gla_fwd_framecausal_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_fwd_framecausal(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in),
                                   _ptr(z_in), _ptr(o), _ptr(S_out), _ptr(z_out), B, H, F, T, d,
                                   dt, eps, _ptr(ws), wsb,

                                   _stream_handle(stream, dev, q, k, v, g, gamma, S_in, z_in, o,
                                                  S_out, z_out, ws)))
    return (o, S_out, z_out) if want_state else o


def gla_fwd_framecausal_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                g: torch.Tensor, gamma: torch.Tensor, out: torch.Tensor,
                                S_in: Optional[torch.Tensor] = None,
                                z_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                S_out: Optional[torch.Tensor] = None,
                                z_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """gla_fwd_framecausal with its workspace in the library's static device
    scratch (NOALLOC_SCRATCH_BYTES per GPU): neither this binding nor the call
    allocates, so the caller passes ``out`` (and S_out, z_out for the state).
    Calls that overlap in time on one GPU race on the scratch."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    _like(out, ref, "out")
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device(q, k, v, g, gamma, S_in, z_in, out, S_out, z_out)
    _check(lib.gla_fwd_framecausal_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in), _ptr(out),
        _ptr(S_out), _ptr(z_out), B, H, F, T, d, dt, eps,
        _stream_handle(stream, dev, q, k, v, g, gamma, S_in, z_in, out, S_out, z_out)))
    return out


def gla_fwd_framecausal_states(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               g: torch.Tensor, gamma: torch.Tensor,
                               S_in: Optional[torch.Tensor] = None,
                               z_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                               out: Optional[torch.Tensor] = None,
                               states: Optional[torch.Tensor] = None,
                               S_out: Optional[torch.Tensor] = None,
                               z_out: Optional[torch.Tensor] = None, return_state: bool = False,
                               workspace: Optional[torch.Tensor] = None, stream=None):
    """gla_fwd_framecausal that also records every frame's state for the backward.

    ``states`` is float32 [B, H, F, d*d + d]: S_f (row-major) then z_f per frame.
    Returns ``(o, states)``, or ``(o, states, S_out, z_out)`` when
    ``return_state`` is set or S_out/z_out are given."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    want_state = return_state or S_out is not None or z_out is not None
    if want_state and S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if want_state and z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    if states is None:
        states = torch.empty((B, H, F, d * d + d), dtype=torch.float32, device=ref.device)
    elif states.shape != (B, H, F, d * d + d) or states.dtype != torch.float32:
        raise ValueError("states must be float32 [B, H, F, d*d + d]")
    o = torch.empty_like(ref) if out is None else out
    _like(o, ref, "out")
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device(q, k, v, g, gamma, S_in, z_in, o, states, S_out, z_out, workspace)
    ws, wsb = _workspace(lib.gla_fwd_framecausal_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_fwd_framecausal_states(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in), _ptr(o),
        _ptr(S_out), _ptr(z_out), _ptr(states), B, H, F, T, d, dt, eps, _ptr(ws), wsb,
        _stream_handle(stream, dev, q, k, v, g, gamma, S_in, z_in, o, states, S_out, z_out,
                       ws)))
    return (o, states, S_out, z_out) if want_state else (o, states)


def gla_state_carry(k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                    S_in: Optional[torch.Tensor] = None, z_in: Optional[torch.Tensor] = None,
                    S_out: Optional[torch.Tensor] = None, z_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """State (S, z) after the frames of k, v: the block KV cache commit."""
    lib = load_library()
    ref = _qkvg(k, v)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    if S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device(k, v, gamma, S_in, z_in, S_out, z_out, workspace)
    ws, wsb = _workspace(lib.gla_state_carry_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_state_carry(_ptr(k), _ptr(v), _ptr(gamma), _ptr(S_in), _ptr(z_in),
                               _ptr(S_out), _ptr(z_out), B, H, F, T, d, dt,
                               _ptr(ws), wsb,
                               _stream_handle(stream, dev, k, v, gamma, S_in, z_in, S_out, z_out,
                                              ws)))
    return S_out, z_out


def gla_fwd_bidir_ex_workspace(B: int, H: int, F: int, T: int, d: int, rope=None) -> int:
    return int(load_library().gla_fwd_bidir_ex_workspace(B, H, F, T, d, _rope(rope)))


def _frames_of(N: int, rope, F: Optional[int]) -> Tuple[int, int]:
    """(F, T) of a bidirectional call: T from the rotary grid, else one frame."""
    if rope is not None:
        r = rope if isinstance(rope, Rope3D) else Rope3D(**rope)
        T = r.grid_h * r.grid_w
        if N % T:
            raise ValueError("N=%d is not a multiple of the grid's %d tokens" % (N, T))
        return N // T, T
    if F:
        if N % F:
            raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
        return F, N // F
    return (1, N) if N else (0, 0)


def gla_fwd_bidir_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     eps: float = 1e-6, rope=None, frames: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """gla_fwd_bidir on [B, H, N, d] views of any layout with a contiguous
    feature axis, optionally with 3D rotary positions (frames of
    grid_h * grid_w tokens). ``out`` defaults to torch.empty_like(q)."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F, T = _frames_of(N, rope, frames)
    o = torch.empty_like(q) if out is None else out
    if o.shape != ref.shape or o.dtype != ref.dtype:
        raise ValueError("out must match q's shape and dtype")
    dev = _require_device_any_layout(q, k, v, g, o, dense=(workspace,))
    ws, wsb = _workspace(lib.gla_fwd_bidir_ex_workspace(B, H, F, T, d, _rope(rope)), dev,
                         workspace)
    _check(lib.gla_fwd_bidir_ex(_view(q), _view(k), _view(v), _view(g), _view(o), B, H, F, T, d,
                                dt, eps, _rope(rope), _ptr(ws), wsb,
                                _stream_handle(stream, dev, q, k, v, g, o, ws)))
    return o


def gla_fwd_framecausal_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                           gamma: torch.Tensor, S_in: Optional[torch.Tensor] = None,
                           z_in: Optional[torch.Tensor] = None, eps: float = 1e-6, rope=None,
                           out: Optional[torch.Tensor] = None,
                           S_out: Optional[torch.Tensor] = None,
                           z_out: Optional[torch.Tensor] = None, return_state: bool = False,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """gla_fwd_framecausal on views of any layout with a contiguous feature
    axis, optionally with 3D rotary positions. ``out`` defaults to
    torch.empty_like(q)."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    want_state = return_state or S_out is not None or z_out is not None
    if want_state and S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if want_state and z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    o = torch.empty_like(q) if out is None else out
    if o.shape != ref.shape or o.dtype != ref.dtype:
        raise ValueError("out must match q's shape and dtype")
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device_any_layout(q, k, v, g, o,
                                     dense=(gamma, S_in, z_in, S_out, z_out, workspace))
    ws, wsb = _workspace(lib.gla_fwd_framecausal_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_fwd_framecausal_ex(_view(q), _view(k), _view(v), _view(g), _ptr(gamma),
                                      _ptr(S_in), _ptr(z_in), _view(o), _ptr(S_out), _ptr(z_out),
                                      B, H, F, T, d, dt, eps, _rope(rope), _ptr(ws), wsb,

                                      _stream_handle(stream, dev, q, k, v, g, gamma, S_in, z_in,
                                                     o, S_out, z_out, ws)))
    return (o, S_out, z_out) if want_state else o


def gla_fwd_framecausal_states_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  g: torch.Tensor, gamma: torch.Tensor,
                                  S_in: Optional[torch.Tensor] = None,
                                  z_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                  rope=None, out: Optional[torch.Tensor] = None,
                                  states: Optional[torch.Tensor] = None,
                                  S_out: Optional[torch.Tensor] = None,
                                  z_out: Optional[torch.Tensor] = None,
                                  return_state: bool = False,
                                  workspace: Optional[torch.Tensor] = None, stream=None):
    """gla_fwd_framecausal_states on views of any layout with a contiguous
    feature axis, optionally with 3D rotary positions (the record then holds
    the turned-key states). Returns ``(o, states)`` or
    ``(o, states, S_out, z_out)``."""
    lib = load_library()
    ref = _qkvg(q, k, v, g)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    want_state = return_state or S_out is not None or z_out is not None
    if want_state and S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if want_state and z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    if states is None:
        states = torch.empty((B, H, F, d * d + d), dtype=torch.float32, device=ref.device)
    elif states.shape != (B, H, F, d * d + d) or states.dtype != torch.float32:
        raise ValueError("states must be float32 [B, H, F, d*d + d]")
    o = torch.empty_like(q) if out is None else out
    if o.shape != ref.shape or o.dtype != ref.dtype:
        raise ValueError("out must match q's shape and dtype")
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device_any_layout(q, k, v, g, o, dense=(gamma, S_in, z_in, states, S_out,
                                                           z_out, workspace))
    ws, wsb = _workspace(lib.gla_fwd_framecausal_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_fwd_framecausal_states_ex(
        _view(q), _view(k), _view(v), _view(g), _ptr(gamma), _ptr(S_in), _ptr(z_in), _view(o),
        _ptr(S_out), _ptr(z_out), _ptr(states), B, H, F, T, d, dt, eps, _rope(rope), _ptr(ws),
        wsb,
        _stream_handle(stream, dev, q, k, v, g, gamma, S_in, z_in, o, states, S_out, z_out, ws)))
    return (o, states, S_out, z_out) if want_state else (o, states)


def gla_state_carry_ex(k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                       S_in: Optional[torch.Tensor] = None, z_in: Optional[torch.Tensor] = None,
                       S_out: Optional[torch.Tensor] = None, z_out: Optional[torch.Tensor] = None,
                       rope=None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gla_state_carry on views of any layout, optionally with rotary positions."""
    lib = load_library()
    ref = _qkvg(k, v)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    if S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    _states(B, H, d, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    dev = _require_device_any_layout(k, v, dense=(gamma, S_in, z_in, S_out, z_out, workspace))
    ws, wsb = _workspace(lib.gla_state_carry_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_state_carry_ex(_view(k), _view(v), _ptr(gamma), _ptr(S_in), _ptr(z_in),
                                  _ptr(S_out), _ptr(z_out), B, H, F, T, d, dt, _rope(rope),
                                  _ptr(ws), wsb,
                                  _stream_handle(stream, dev, k, v, gamma, S_in, z_in, S_out,
                                                 z_out, ws)))
    return S_out, z_out


def gla_bwd_framecausal_workspace(B: int, H: int, F: int, T: int, d: int) -> int:
    return int(load_library().gla_bwd_framecausal_workspace(B, H, F, T, d))


def gla_bwd_bidir_workspace(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().gla_bwd_bidir_workspace(B, H, N, d))


def gla_bwd_framecausal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        gamma: torch.Tensor, dO: torch.Tensor,
                        S_in: Optional[torch.Tensor] = None, z_in: Optional[torch.Tensor] = None,
                        dS_out: Optional[torch.Tensor] = None,
                        dz_out: Optional[torch.Tensor] = None, eps: float = 1e-6,
                        need_state_grad: Optional[bool] = None, out: Optional[dict] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of gla_fwd_framecausal for dL/do = dO (and dL/dS_out, dL/dz_out).

    Returns {"dq", "dk", "dv", "dg", "dgamma"} and, when ``need_state_grad``
    (default: S_in or dS_out given), "dS_in" and "dz_in". ``out`` may supply
    any of these tensors to be written."""
    return _bwd_framecausal(q, k, v, g, gamma, None, dO, S_in, z_in, dS_out, dz_out, eps,
                            need_state_grad, out, workspace, stream)


def gla_bwd_framecausal_states(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               g: torch.Tensor, gamma: torch.Tensor, states: torch.Tensor,
                               dO: torch.Tensor, S_in: Optional[torch.Tensor] = None,
                               z_in: Optional[torch.Tensor] = None,
                               dS_out: Optional[torch.Tensor] = None,
                               dz_out: Optional[torch.Tensor] = None, eps: float = 1e-6,
                               need_state_grad: Optional[bool] = None,
                               out: Optional[dict] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """gla_bwd_framecausal given the states recorded by gla_fwd_framecausal_states
    for the same inputs (no recompute; bitwise the same gradients)."""
    return _bwd_framecausal(q, k, v, g, gamma, states, dO, S_in, z_in, dS_out, dz_out, eps,
                            need_state_grad, out, workspace, stream)


def gla_bwd_framecausal_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                           gamma: torch.Tensor, dO: torch.Tensor,
                           states: Optional[torch.Tensor] = None,
                           S_in: Optional[torch.Tensor] = None,
                           z_in: Optional[torch.Tensor] = None,
                           dS_out: Optional[torch.Tensor] = None,
                           dz_out: Optional[torch.Tensor] = None, eps: float = 1e-6,
                           rope=None, need_state_grad: Optional[bool] = None,
                           out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> dict:
    """The frame-causal backward on views of any layout with a contiguous
    feature axis (e.g. q, k, v slices of a fused [B, N, 3, H, d] projection),
    optionally with 3D rotary positions (the gradients of
    gla_fwd_framecausal_ex with the same ``rope``); ``states``: the record of
    gla_fwd_framecausal_states(_ex) for the same inputs and rope, or None to
    recompute. ``out`` may supply dq, dk, dv, dg (views too; they may not
    overlap one another) and the fp32 gradients; missing ones are allocated
    contiguous."""
    lib = load_library()
    ref = _qkvg(q, k, v, g, dO)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    if states is not None and (states.shape != (B, H, F, d * d + d)
                               or states.dtype != torch.float32):
        raise ValueError("states must be float32 [B, H, F, d*d + d]")
    if need_state_grad is None:
        need_state_grad = S_in is not None or dS_out is not None
    out = dict(out or {})
    for n in ("dq", "dk", "dv", "dg"):
        out.setdefault(n, torch.empty(ref.shape, dtype=ref.dtype, device=ref.device))
        if out[n].shape != ref.shape or out[n].dtype != ref.dtype:
            raise ValueError("%s must match q's shape and dtype" % n)
    out.setdefault("dgamma", torch.empty((B, H, F), dtype=torch.float32, device=ref.device))
    if need_state_grad:
        out.setdefault("dS_in", torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device))
        out.setdefault("dz_in", torch.empty((B, H, d), dtype=torch.float32, device=ref.device))
    _states(B, H, d, S_in=S_in, z_in=z_in, dS_out=dS_out, dz_out=dz_out,
            dS_in=out.get("dS_in"), dz_in=out.get("dz_in"))
    _dense(out["dgamma"], (B, H, F), "dgamma")
    dev = _require_device_any_layout(
        q, k, v, g, dO, out["dq"], out["dk"], out["dv"], out["dg"],
        dense=(gamma, states, S_in, z_in, dS_out, dz_out, out["dgamma"], out.get("dS_in"),
               out.get("dz_in"), workspace))
    if states is None:
        nbytes = lib.gla_bwd_framecausal_workspace(B, H, F, T, d)
    else:
        nbytes = lib.gla_bwd_framecausal_states_workspace(B, H, F, T, d)
    ws, wsb = _workspace(nbytes, dev, workspace)
    _check(lib.gla_bwd_framecausal_ex(
        _view(q), _view(k), _view(v), _view(g), _ptr(gamma), _ptr(S_in), _ptr(z_in), _ptr(states),
        _view(dO), _ptr(dS_out), _ptr(dz_out), _view(out["dq"]), _view(out["dk"]),
        _view(out["dv"]), _view(out["dg"]), _ptr(out["dgamma"]), _ptr(out.get("dS_in")),
        _ptr(out.get("dz_in")), B, H, F, T, d, dt, eps, _rope(rope), _ptr(ws), wsb,
        _stream_handle(stream, dev, q, k, v, g, gamma, states, S_in, z_in, dO, dS_out, dz_out,
                       out, ws)))
    return out


def gla_bwd_bidir_ex_workspace(B: int, H: int, F: int, T: int, d: int, rope=None) -> int:
    return int(load_library().gla_bwd_bidir_ex_workspace(B, H, F, T, d, _rope(rope)))


def gla_bwd_bidir_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     dO: torch.Tensor, eps: float = 1e-6, rope=None,
                     frames: Optional[int] = None, out: Optional[dict] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of gla_fwd_bidir_ex (same ``rope`` and ``frames``) for
    dL/do = dO on views of any layout with a contiguous feature axis:
    {"dq", "dk", "dv", "dg"}; ``out`` may supply any of them (views too)."""
    lib = load_library()
    ref = _qkvg(q, k, v, g, dO)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F, T = _frames_of(N, rope, frames)
    out = dict(out or {})
    for n in ("dq", "dk", "dv", "dg"):
        out.setdefault(n, torch.empty(ref.shape, dtype=ref.dtype, device=ref.device))
        if out[n].shape != ref.shape or out[n].dtype != ref.dtype:
            raise ValueError("%s must match q's shape and dtype" % n)
    dev = _require_device_any_layout(q, k, v, g, dO, out["dq"], out["dk"], out["dv"],
                                     out["dg"], dense=(workspace,))
    ws, wsb = _workspace(lib.gla_bwd_bidir_ex_workspace(B, H, F, T, d, _rope(rope)), dev,
                         workspace)
    _check(lib.gla_bwd_bidir_ex(_view(q), _view(k), _view(v), _view(g), _view(dO),
                                _view(out["dq"]), _view(out["dk"]), _view(out["dv"]),
                                _view(out["dg"]), B, H, F, T, d, dt, eps, _rope(rope), _ptr(ws),
                                wsb, _stream_handle(stream, dev, q, k, v, g, dO, out, ws)))
    return out


def gla_bwd_framecausal_states_workspace(B: int, H: int, F: int, T: int, d: int) -> int:
    return int(load_library().gla_bwd_framecausal_states_workspace(B, H, F, T, d))


def _bwd_framecausal(q, k, v, g, gamma, states, dO, S_in, z_in, dS_out, dz_out, eps,
                     need_state_grad, out, workspace, stream) -> dict:
    lib = load_library()
    ref = _qkvg(q, k, v, g, dO)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    if states is not None and (states.shape != (B, H, F, d * d + d)
                               or states.dtype != torch.float32):
        raise ValueError("states must be float32 [B, H, F, d*d + d]")
    if need_state_grad is None:
        need_state_grad = S_in is not None or dS_out is not None
    out = dict(out or {})
    for n in ("dq", "dk", "dv", "dg"):
        out.setdefault(n, torch.empty_like(ref))
    out.setdefault("dgamma", torch.empty((B, H, F), dtype=torch.float32, device=ref.device))
    if need_state_grad:
        out.setdefault("dS_in", torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device))
        out.setdefault("dz_in", torch.empty((B, H, d), dtype=torch.float32, device=ref.device))
    for n in ("dq", "dk", "dv", "dg"):
        _like(out[n], ref, n)
    _states(B, H, d, S_in=S_in, z_in=z_in, dS_out=dS_out, dz_out=dz_out,
            dS_in=out.get("dS_in"), dz_in=out.get("dz_in"))
    _dense(out["dgamma"], (B, H, F), "dgamma")
    dev = _require_device(q, k, v, g, gamma, states, dO, S_in, z_in, dS_out, dz_out, workspace,
                          *out.values())
    grads = (_ptr(dO), _ptr(dS_out), _ptr(dz_out), _ptr(out["dq"]), _ptr(out["dk"]),
             _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dgamma"]), _ptr(out.get("dS_in")),
             _ptr(out.get("dz_in")))
    if states is None:
        nbytes = lib.gla_bwd_framecausal_workspace(B, H, F, T, d)
    else:
        nbytes = lib.gla_bwd_framecausal_states_workspace(B, H, F, T, d)
    ws, wsb = _workspace(nbytes, dev, workspace)
    handle = _stream_handle(stream, dev, q, k, v, g, gamma, states, S_in, z_in, dO, dS_out,
                            dz_out, out, ws)
    if states is None:
        _check(lib.gla_bwd_framecausal(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in), *grads,
            B, H, F, T, d, dt, eps, _ptr(ws), wsb, handle))
    else:
        _check(lib.gla_bwd_framecausal_states(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(S_in), _ptr(z_in),
            _ptr(states), *grads, B, H, F, T, d, dt, eps, _ptr(ws), wsb, handle))
    return out


def gla_bwd_bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  dO: torch.Tensor, eps: float = 1e-6, out: Optional[dict] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of gla_fwd_bidir for dL/do = dO: {"dq", "dk", "dv", "dg"}."""
    lib = load_library()
    ref = _qkvg(q, k, v, g, dO)
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    out = dict(out or {})
    for n in ("dq", "dk", "dv", "dg"):
        out.setdefault(n, torch.empty_like(ref))
    for n in ("dq", "dk", "dv", "dg"):
        _like(out[n], ref, n)
    dev = _require_device(q, k, v, g, dO, workspace, *out.values())
    ws, wsb = _workspace(lib.gla_bwd_bidir_workspace(B, H, N, d), dev, workspace)
    _check(lib.gla_bwd_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dO), _ptr(out["dq"]),
                             _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), B, H, N, d, dt,
                             eps, _ptr(ws), wsb,
                             _stream_handle(stream, dev, q, k, v, g, dO, out, ws)))
    return out


def gla_gdn_framecausal_workspace(B: int, H: int, F: int, T: int, d: int) -> int:
    return int(load_library().gla_gdn_framecausal_workspace(B, H, F, T, d))


def gla_gdn_framecausal(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                        beta: torch.Tensor, gamma: torch.Tensor,
                        S_in: Optional[torch.Tensor] = None, key_scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, S_out: Optional[torch.Tensor] = None,
                        return_state: bool = False, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """Frame-wise Gated DeltaNet: F = gamma.shape[-1], T = N / F; beta [B, H, N]
    fp32. key_scale defaults to 1/sqrt(d T). q None computes the state only.

    Returns o, or (o, S_out) with ``return_state`` or S_out given."""
    lib = load_library()
    ref = _qkvg(*(t for t in (q, k, v) if t is not None))
    dt = _dtype_code(ref)
    B, H, N, d = ref.shape
    F = int(gamma.shape[-1])
    if gamma.shape != (B, H, F) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be float32 [B, H, F]")
    if beta.shape != (B, H, N) or beta.dtype != torch.float32:
        raise ValueError("beta must be float32 [B, H, N]")
    if (F == 0 and N != 0) or (F and N % F):
        raise ValueError("N=%d is not a multiple of F=%d" % (N, F))
    T = N // F if F else 0
    if key_scale is None:
        key_scale = 1.0 / (d * T) ** 0.5 if T else 1.0
    want_state = return_state or S_out is not None or q is None
    if want_state and S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    o = None if q is None else (torch.empty_like(ref) if out is None else out)
    if o is not None:
        _like(o, ref, "out")
    _dense(S_in, (B, H, d, d), "S_in")
    _dense(S_out, (B, H, d, d), "S_out")
    dev = _require_device(q, k, v, beta, gamma, S_in, o, S_out, workspace)
    ws, wsb = _workspace(lib.gla_gdn_framecausal_workspace(B, H, F, T, d), dev, workspace)
    _check(lib.gla_gdn_framecausal(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma),
                                   _ptr(S_in), _ptr(o), _ptr(S_out), B, H, F, T, d, dt,
                                   float(key_scale), _ptr(ws), wsb,
                                   _stream_handle(stream, dev, q, k, v, beta, gamma, S_in, o,
                                                  S_out, ws)))
    if q is None:
        return S_out
    return (o, S_out) if want_state else o


def gla_softmax_anchor(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                       T: int, causal: bool = True, n_sink: int = 0, window: int = 0,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Gated softmax attention over whole frames: o = sigmoid(g) * softmax(scale q k^T) v.

    k, v [B, H, F*T, d]; q, g [B, H, Fq*T, d], the tokens of the last Fq key
    frames. causal False: every key visible. causal True: query frame f sees
    key frames i <= f with i < n_sink or i > f - window (window <= 0: no
    limit). scale defaults to 1/sqrt(d)."""
    lib = load_library()
    if k.dim() != 4 or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must be [B, H, F*T, d] of one dtype")
    if q.dim() != 4 or g.shape != q.shape or q.dtype != k.dtype or g.dtype != k.dtype \
            or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q and g must be [B, H, Fq*T, d] in k's dtype")
    B, H, Nk, d = k.shape
    Nq = q.shape[2]
    if T <= 0 or Nk % T or Nq % T or Nq > Nk:
        raise ValueError("Nq=%d and Nk=%d must be multiples of T=%d with Nq <= Nk" % (Nq, Nk, T))
    if scale is None:
        scale = 1.0 / d ** 0.5
    o = torch.empty_like(q) if out is None else out
    _like(o, q, "out")
    dev = _require_device(q, k, v, g, o)
    _check(lib.gla_softmax_anchor(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), B, H, Nq // T,
                                  Nk // T, T, d, _dtype_code(k), int(bool(causal)), int(n_sink),
                                  int(window), float(scale),
                                  _stream_handle(stream, dev, q, k, v, g, o)))
    return o


PROBE_KINDS = ("read", "read_nt", "write", "write_nt", "copy", "copy_nt", "read2_write1",
               "read2_write1_nt", "read2_nt_write_eighth")


def stream_probe(kind: str, out: torch.Tensor, a: Optional[torch.Tensor] = None,
                 b: Optional[torch.Tensor] = None, stream=None) -> None:
    """One launch of the library's bandwidth probe (``gla_stream_probe``) over
    ``out.numel() * out.element_size()`` bytes; kind is one of PROBE_KINDS."""
    lib = load_library()
    nbytes = out.numel() * out.element_size()
    for t in (a, b):
        if t is not None and t.numel() * t.element_size() != nbytes:
            raise ValueError("probe buffers must have equal sizes")
    dev = _require_device(out, a, b)
    _check(lib.gla_stream_probe(PROBE_KINDS.index(kind), _ptr(a), _ptr(b), _ptr(out), nbytes,
                                _stream_handle(stream, dev, out, a, b)))


def profile_begin(max_launches: int = 4096) -> None:
    """Start timing every kernel the entry points launch (HIP events on their stream)."""
    _check(load_library().gla_profile_begin(int(max_launches)))


def profile_end() -> dict:
    """Stop timing; returns {kernel kind: (launches, summed milliseconds)}."""
    lib = load_library()
    cap = 16  # more than the library's kernel kinds
    out = (_KernelTime * cap)()
    n = ctypes.c_int(0)
    _check(lib.gla_profile_end(out, cap, ctypes.byref(n)))
    return {out[i].name.decode(): (out[i].launches, out[i].total_ms)
            for i in range(min(n.value, cap))}
