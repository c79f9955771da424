"""The gated linear-attention mixer as ``torch.autograd`` functions.

Both directions run in ``libgla.so``: the forward through
:func:`gla_fwd_framecausal_states_ex` (or :func:`gla_fwd_framecausal_ex`) and
:func:`gla_fwd_bidir_ex`, the backward through :func:`gla_bwd_framecausal_ex`
and :func:`gla_bwd_bidir_ex`. These classes only route tensors between
autograd and those calls. q, k, v, g may be any [B, H, N, d] views with a
contiguous feature axis (e.g. slices of a fused projection): neither direction
copies them. Both modes take optional 3D rotary positions (``rope``: a
:class:`Rope3D` or its fields as a dict), with which the gradients are those
of the rotary form.

Frame-causal mode keeps, by default, every frame's state from the forward
([B, H, F, d*d + d] float32, 128 MB per call at the 720p/60s shape with
H = 32, d = 64) so that the backward need not recompute it; pass
``save_states=False`` to recompute instead and keep only the inputs.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (gla_bwd_bidir_ex, gla_bwd_framecausal_ex, gla_fwd_bidir_ex,
               gla_fwd_framecausal_ex, gla_fwd_framecausal_states_ex)

__all__ = ["FrameCausal", "Bidirectional", "gla_framecausal", "gla_bidir"]


class FrameCausal(torch.autograd.Function):
    """(q, k, v, g, gamma, S_in, z_in) -> (o, S_out, z_out), frame-causal."""

    @staticmethod
    def forward(ctx, q, k, v, g, gamma, S_in, z_in, eps: float, save_states: bool, rope):
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        if save_states:
            o, states, S_out, z_out = gla_fwd_framecausal_states_ex(
                q, k, v, g, gamma, S_in, z_in, eps=eps, rope=rope, out=out, return_state=True)
        else:
            o, S_out, z_out = gla_fwd_framecausal_ex(q, k, v, g, gamma, S_in, z_in, eps=eps,
                                                     rope=rope, out=out, return_state=True)
            states = None
        ctx.save_for_backward(q, k, v, g, gamma, S_in, z_in, states)
        ctx.eps = eps
        ctx.rope = rope
        ctx.set_materialize_grads(False)
        return o, S_out, z_out

    @staticmethod
    def backward(ctx, dO, dS_out, dz_out):
        q, k, v, g, gamma, S_in, z_in, states = ctx.saved_tensors
        if dO is None:
            dO = torch.zeros_like(q)
        # the call takes both state gradients or neither
        B, H, d = q.shape[0], q.shape[1], q.shape[-1]
        if dS_out is None and dz_out is not None:
            dS_out = torch.zeros((B, H, d, d), dtype=torch.float32, device=q.device)
        if dz_out is None and dS_out is not None:
            dz_out = torch.zeros((B, H, d), dtype=torch.float32, device=q.device)
        # a loss that reduces the state (S_out.sum(), z_out.mean()) hands over
        # expanded gradients with zero strides; the call reads dense arrays
        if dS_out is not None:
            dS_out, dz_out = dS_out.contiguous(), dz_out.contiguous()
        need_state = S_in is not None and (ctx.needs_input_grad[5] or ctx.needs_input_grad[6])
        grads = gla_bwd_framecausal_ex(q, k, v, g, gamma, dO.contiguous(), states=states,
                                       S_in=S_in, z_in=z_in, dS_out=dS_out, dz_out=dz_out,
                                       eps=ctx.eps, rope=ctx.rope, need_state_grad=need_state)
        return (grads["dq"], grads["dk"], grads["dv"], grads["dg"], grads["dgamma"],
                grads.get("dS_in"), grads.get("dz_in"), None, None, None)


class Bidirectional(torch.autograd.Function):
    """(q, k, v, g) -> o with one state over the whole sequence."""

    @staticmethod
    def forward(ctx, q, k, v, g, eps: float, rope, frames):
        ctx.save_for_backward(q, k, v, g)
        ctx.eps = eps
        ctx.rope = rope
        ctx.frames = frames
        return gla_fwd_bidir_ex(q, k, v, g, eps=eps, rope=rope, frames=frames,
                                out=torch.empty(q.shape, dtype=q.dtype, device=q.device))

    @staticmethod
    def backward(ctx, dO):
        q, k, v, g = ctx.saved_tensors
        grads = gla_bwd_bidir_ex(q, k, v, g, dO.contiguous(), eps=ctx.eps, rope=ctx.rope,
                                 frames=ctx.frames)
        return grads["dq"], grads["dk"], grads["dv"], grads["dg"], None, None, None


def gla_framecausal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    gamma: torch.Tensor, S_in: Optional[torch.Tensor] = None,
                    z_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                    save_states: bool = True, return_state: bool = False, rope=None):
    """Differentiable frame-causal gated linear attention (q, k, v, g any
    [B, H, F*T, d] views with a contiguous feature axis; gamma float32
    [B, H, F]; optional carried S_in, z_in; optional 3D rotary positions).

    Returns o, or (o, S_out, z_out) with ``return_state``; gradients reach q,
    k, v, g, gamma and S_in, z_in."""
    o, S_out, z_out = FrameCausal.apply(q, k, v, g, gamma, S_in, z_in, eps, save_states, rope)
    return (o, S_out, z_out) if return_state else o


def gla_bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              eps: float = 1e-6, rope=None, frames: Optional[int] = None) -> torch.Tensor:
    """Differentiable bidirectional gated linear attention (q, k, v, g any
    [B, H, N, d] views with a contiguous feature axis), optionally with 3D
    rotary positions over frames of grid_h * grid_w tokens."""
    return Bidirectional.apply(q, k, v, g, eps, rope, frames)
