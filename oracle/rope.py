"""NeoX (split-half) and interleaved rotary position embedding (oracle only).

The pages name the operation but print no formula: Loom Kernels lists a
NeoX or interleaved RoPE fused with the native or static-FP8 paged-KV write
among its supported operator paths (row «Position and KV»), and
microLLM-rocm's ledger names the same layout as the split-half form.  The
textbook split-half rotary embedding is taken: for a
head vector x of even length D, pair i (0 <= i < D/2) is (x[i], x[i + D/2]),
rotated by the angle pos * w_i with w_i = theta ** (-2i/D):

    y[i]       = x[i] * cos - x[i + D/2] * sin
    y[i + D/2] = x[i + D/2] * cos + x[i] * sin

The interleaved form (the GPT-J layout; Loom's "interleaved RoPE") pairs
adjacent elements instead: pair i is (x[2i], x[2i + 1]) with the same angle
pos * w_i:

    y[2i]     = x[2i] * cos - x[2i + 1] * sin
    y[2i + 1] = x[2i + 1] * cos + x[2i] * sin

Two evaluations are provided for each:
  rope_neox_f64        the exact rotation in fp64 (the mathematical result);
  rope_neox_f32_recipe the rotation as a device evaluates it in fp32: the
                       angle and its cosine/sine in fp64, each rounded once to
                       fp32, then every product and difference rounded to fp32
                       on its own (no fused multiply-add).  NumPy float32
                       arithmetic never fuses, so this is that recipe exactly.
"""
from __future__ import annotations

import numpy as np


def rope_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """w_i = theta ** (-2i / D) for i in [0, D/2), in fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(head_dim))


def rope_angles(pos, theta: float, head_dim: int) -> np.ndarray:
    """pos * w_i in fp64; pos may be an array (broadcast on a leading axis)."""
    pos = np.asarray(pos, dtype=np.float64)
    return pos[..., None] * rope_inv_freq(theta, head_dim)


def _per_row(a: np.ndarray, x_ndim: int) -> np.ndarray:
    """Reshape angles [B, D/2] to [B, 1, ..., 1, D/2] so they broadcast over
    an x of shape [B, ..., D]; a scalar position gives [D/2] unchanged."""
    if a.ndim == 1:
        return a
    return a.reshape((a.shape[0],) + (1,) * (x_ndim - 2) + (a.shape[-1],))


def rope_neox_f64(x, pos, theta: float) -> np.ndarray:
    """Exact split-half rotation of x[..., D] (fp64).  ``pos`` is a scalar or
    one position per row of x's first axis."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = _per_row(rope_angles(pos, theta, D), x.ndim)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_cos_sin_f32(pos, theta: float, head_dim: int):
    """cos and sin of the fp64 angle, each rounded once to fp32."""
    ang = rope_angles(pos, theta, head_dim)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_neox_f32_recipe(x, pos, theta: float) -> np.ndarray:
    """The fp32 evaluation recipe of the same rotation (see module doc)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    half = D // 2
    c, s = rope_cos_sin_f32(pos, theta, D)
    c, s = _per_row(c, x.ndim), _per_row(s, x.ndim)
    lo, hi = x[..., :half], x[..., half:]
    f32 = np.float32
    y_lo = np.subtract(np.multiply(lo, c, dtype=f32), np.multiply(hi, s, dtype=f32), dtype=f32)
    y_hi = np.add(np.multiply(hi, c, dtype=f32), np.multiply(lo, s, dtype=f32), dtype=f32)
    return np.concatenate([y_lo, y_hi], axis=-1)


def rope_interleaved_f64(x, pos, theta: float) -> np.ndarray:
    """Exact adjacent-pair rotation of x[..., D] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = _per_row(rope_angles(pos, theta, D), x.ndim)
    c, s = np.cos(ang), np.sin(ang)
    ev, od = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = ev * c - od * s
    y[..., 1::2] = od * c + ev * s
    return y


def rope_interleaved_f32_recipe(x, pos, theta: float) -> np.ndarray:
    """The fp32 evaluation recipe of the adjacent-pair rotation."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    c, s = rope_cos_sin_f32(pos, theta, D)
    c, s = _per_row(c, x.ndim), _per_row(s, x.ndim)
    ev, od = x[..., 0::2], x[..., 1::2]
    f32 = np.float32
    y = np.empty_like(x)
    y[..., 0::2] = np.subtract(np.multiply(ev, c, dtype=f32), np.multiply(od, s, dtype=f32), dtype=f32)
    y[..., 1::2] = np.add(np.multiply(od, c, dtype=f32), np.multiply(ev, s, dtype=f32), dtype=f32)
    return y


ROPE_STYLES = ("neox", "interleaved")


def rope_f64(x, pos, theta: float, style: str = "neox") -> np.ndarray:
    if style == "neox":
        return rope_neox_f64(x, pos, theta)
    if style == "interleaved":
        return rope_interleaved_f64(x, pos, theta)
    raise ValueError(style)


def rope_f32_recipe(x, pos, theta: float, style: str = "neox") -> np.ndarray:
    if style == "neox":
        return rope_neox_f32_recipe(x, pos, theta)
    if style == "interleaved":
        return rope_interleaved_f32_recipe(x, pos, theta)
    raise ValueError(style)
