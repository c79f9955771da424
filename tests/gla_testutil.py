"""Shared helpers for the test suite (comparison metric, small input builders)."""
from __future__ import annotations

import numpy as np

# Tolerances of the parity bar: fp32 inputs and bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def slab_rel_err(o: np.ndarray, ref: np.ndarray) -> float:
    """max_i |o_i - r_i| / max(|r_i|, rms of r over the (b, h) slab).

    Outputs are normalised averages of many signed values and sit close to zero,
    so a pure elementwise relative error is dominated by near-zero references;
    the slab rms floors the denominator. Arrays are [B, H, N, d] (or any shape
    whose last two axes form the slab)."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    lead = ref.shape[:-2] if ref.ndim >= 2 else ()
    r2 = ref.reshape(lead + (-1,)) if lead else ref.reshape(1, -1)
    o2 = o.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
    denom = np.maximum(np.abs(r2), rms)
    denom = np.where(denom == 0, 1.0, denom)
    err = np.abs(o2 - r2) / denom
    if not np.all(np.isfinite(o2)):
        return float("inf")
    return float(err.max())


def max_abs_over_max(o, ref) -> float:
    """max |o - r| / max |r| (reported alongside the slab metric)."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.abs(ref).max() if ref.size else 0.0
    return float(np.abs(o - ref).max() / m) if m > 0 else float(np.abs(o - ref).max())


def close(a, b, rtol=1e-12):
    """|a - b| <= rtol * max|b| elementwise (scale-aware equality for fp64 forms)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.abs(b).max() if b.size else 0.0, 1e-300)
    return bool(np.all(np.abs(a - b) <= rtol * scale))
