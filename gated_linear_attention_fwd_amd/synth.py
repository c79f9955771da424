"""Seeded synthetic inputs for the gated linear-attention forward pass.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic. Both the GPU library's tests and the
CPU oracle are fed from here, so they see the same bits.

Workloads take the latent-video shape of the 720p clips described by the
"SANA-Video 2.0 5B 720p 4-step preview" Space (736x1280 video, 81 frames at
16 FPS): a 32x spatial compression gives a 23 x 40 = 920-token latent frame,
a 4x temporal one gives 21 latent frames for 5 s and 241 for 60 s. Heads and
head dimension are not given by the pages and are assumed.

Recipe (all draws from ``numpy.random.default_rng``):
  * q, k, v, g: float32 ``standard_normal`` in that order, each [B, H, N, d];
    q, k, v (not g) are multiplied by 1/sqrt(d) when ``scale_qkv`` is set;
  * the per-frame decay gamma = 1 / (1 + exp(-x)), x ~ N(mu, sd), [B, H, F],
    drawn after g and stored as float32;
  * bfloat16 storage is round-to-nearest-even of the float32 draw and is held
    as uint16 bit patterns (torch views them as ``torch.bfloat16``).
The streaming workload draws gamma for all frames first from ``seed`` and then
each block's q, k, v, g from the seed sequence ``(seed, block + 1)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

LATENT_GRID_720P = (23, 40)  # latent rows x columns of a 736 x 1280 frame at 32x compression
LATENT_TOKENS_720P = LATENT_GRID_720P[0] * LATENT_GRID_720P[1]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, distributions and seed."""
    name: str
    B: int
    H: int
    d: int
    F: int
    T: int
    dtype: str  # "f32" or "bf16"
    seed: int
    gamma_mu: float
    gamma_sd: float
    scale_qkv: bool
    modes: Tuple[str, ...]
    eps: float = 1e-6
    blocks: Tuple[int, ...] = field(default_factory=tuple)  # frames per streamed block

    @property
    def N(self) -> int:
        return self.F * self.T

    def token_heads(self) -> int:
        return self.B * self.H * self.N

    def io_bytes(self) -> int:
        """Bytes that must cross HBM: read q, k, v, g once and write o once."""
        es = 4 if self.dtype == "f32" else 2
        return 5 * self.token_heads() * self.d * es


WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_oracle_check_B1H2d16_F4T16_f32", 1, 2, 16, 4, 16, "f32", 1001, 2.0, 0.5,
                False, ("bidir", "framecausal")),
    2: Workload("small_B1H8d64_F5T256_bf16", 1, 8, 64, 5, 256, "bf16", 1002, 3.0, 0.5, False,
                ("framecausal",)),
    3: Workload("720p_5s_B1H32d64_F21T920_bf16", 1, 32, 64, 21, LATENT_TOKENS_720P, "bf16", 1003,
                3.0, 0.5, True, ("bidir", "framecausal")),
    4: Workload("720p_60s_B1H32d64_F241T920_bf16", 1, 32, 64, 241, LATENT_TOKENS_720P, "bf16",
                1004, 3.0, 0.5, True, ("framecausal",)),
    5: Workload("720p_60s_streaming_8blocks_B2H40d128_F241T920_bf16", 2, 40, 128, 241,
                LATENT_TOKENS_720P, "bf16", 1005, 2.0, 1.0, True, ("framecausal",),
                blocks=(30, 30, 30, 30, 30, 30, 30, 31)),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite by construction (normal draws), so no NaN handling."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """float32 value of bfloat16 bit patterns (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, scale: float, dtype: str,
          chunk: int = 1 << 24) -> np.ndarray:
    """standard_normal draws of ``shape``, scaled, stored as ``dtype``.

    Drawn in pieces of ``chunk`` values to bound host memory; the sequence is the
    same as one draw of the whole size."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = x if dtype == "f32" else bf16_bits(x)
    return out.reshape(shape)


def _gamma(rng: np.random.Generator, shape, mu: float, sd: float) -> np.ndarray:
    x = rng.normal(mu, sd, size=shape)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def random_inputs(B: int, H: int, F: int, T: int, d: int, dtype: str = "bf16", seed: int = 0,
                  scale_qkv: bool = False, gamma_mu: float = 2.0, gamma_sd: float = 0.5):
    """q, k, v, g ([B,H,F*T,d], float32 or bf16 bits) and gamma ([B,H,F], float32)."""
    rng = np.random.default_rng(seed)
    N = F * T
    s = 1.0 / np.sqrt(d) if scale_qkv else 1.0
    q = _draw(rng, (B, H, N, d), s, dtype)
    k = _draw(rng, (B, H, N, d), s, dtype)
    v = _draw(rng, (B, H, N, d), s, dtype)
    g = _draw(rng, (B, H, N, d), 1.0, dtype)
    gamma = _gamma(rng, (B, H, F), gamma_mu, gamma_sd)
    return dict(q=q, k=k, v=v, g=g, gamma=gamma)


def workload_inputs(w: Workload):
    """Inputs of a one-shot workload (all frames in one call)."""
    return random_inputs(w.B, w.H, w.F, w.T, w.d, w.dtype, w.seed, w.scale_qkv, w.gamma_mu,
                         w.gamma_sd)


def stream_gamma(w: Workload) -> np.ndarray:
    """Decay of every frame of a streamed workload, [B, H, F] float32."""
    return _gamma(np.random.default_rng(w.seed), (w.B, w.H, w.F), w.gamma_mu, w.gamma_sd)


def stream_block_bounds(w: Workload) -> List[Tuple[int, int]]:
    """(first frame, frame count) of every block of a streamed workload."""
    out, f0 = [], 0
    for nf in w.blocks:
        out.append((f0, nf))
        f0 += nf
    assert f0 == w.F
    return out


def stream_block_inputs(w: Workload, block: int, gamma_all: Optional[np.ndarray] = None):
    """q, k, v, g of one streamed block ([B,H,nf*T,d]) and its slice of gamma."""
    f0, nf = stream_block_bounds(w)[block]
    rng = np.random.default_rng((w.seed, block + 1))
    N = nf * w.T
    s = 1.0 / np.sqrt(w.d) if w.scale_qkv else 1.0
    q = _draw(rng, (w.B, w.H, N, w.d), s, w.dtype)
    k = _draw(rng, (w.B, w.H, N, w.d), s, w.dtype)
    v = _draw(rng, (w.B, w.H, N, w.d), s, w.dtype)
    g = _draw(rng, (w.B, w.H, N, w.d), 1.0, w.dtype)
    if gamma_all is None:
        gamma_all = stream_gamma(w)
    gamma = np.ascontiguousarray(gamma_all[:, :, f0:f0 + nf])
    return dict(q=q, k=k, v=v, g=g, gamma=gamma)


def device_inputs(w: Workload, device, block: Optional[int] = None):
    """Inputs drawn on the GPU (torch's Philox generator), for the two workloads
    whose host draw would take minutes: q, k, v, g as torch tensors on
    ``device`` in the workload dtype, gamma as float32 [B, H, F_block].

    Seed: ``seed * 1000`` for a one-shot call, ``seed * 1000 + block + 1`` for
    a streamed block; the draw order is q, k, v, g; gamma is the host draw of
    :func:`stream_gamma` (sliced to the block). Same distributions as the host
    recipe, different random numbers."""
    import torch

    if block is None:
        f0, nf = 0, w.F
        tag = 0
    else:
        f0, nf = stream_block_bounds(w)[block]
        tag = block + 1
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed * 1000 + tag)
    shape = (w.B, w.H, nf * w.T, w.d)
    s = 1.0 / float(np.sqrt(w.d)) if w.scale_qkv else 1.0
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    def draw(scale):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x if tdt == torch.float32 else x.to(tdt)

    q = draw(s)
    k = draw(s)
    v = draw(s)
    g = draw(1.0)
    gamma = torch.from_numpy(np.ascontiguousarray(stream_gamma(w)[:, :, f0:f0 + nf])).to(device)
    return dict(q=q, k=k, v=v, g=g, gamma=gamma)
