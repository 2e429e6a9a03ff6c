"""Fused NeoX RoPE + paged-KV append of the new token (oracle only).

Loom Kernels' supported operator paths include a fused "NeoX/interleaved
RoPE + native/static-FP8 paged-KV write" over packed QKV into NHD cache views
with static per-tensor or per-head FP8 E4M3 scales; its "Next value program"
section adds that the FP8 form writes exact E4M3 bytes.  The pages leave the
details open; the readings taken here are:

* packed QKV row b = [Q heads 0..Hq-1 | K heads 0..Hkv-1 | V heads 0..Hkv-1],
  each head_dim-contiguous;
* context_lens[b] counts the new token, so it is written at position
  pos = ctx - 1: logical block pos // bs, slot pos % bs, physical block
  block_tables[b, pos // bs], and RoPE uses the same position;
* Q and K are rotated, V is stored as is; the rotated Q goes to q_out in the
  activation dtype;
* FP8: code = E4M3(y / scale[g]) with an fp32 division, rounded to nearest
  even, saturating (codecs.e4m3_encode);
* FP4 (mainarch README, decode-attention section: E2M1 KV with E8M0 block
  scales): each 32-element block of the row is quantised with the MX rule of
  codecs.mx_fp4_quantize (scale exponent floor(log2 amax) - 2, codes rounded
  to nearest even and saturating at 6); the division by a power-of-two scale
  is exact, so the recipe needs no fp32 step of its own.  Codes go to the
  block's code area and the scale bytes to its scale area (codecs.fp4_block_views);
* a sequence with ctx <= 0 is inactive: nothing is written to the caches and
  its q_out row is its Q rotated by angle zero, i.e. copied;
* contract variants (Loom's "Position and KV" row: NeoX/interleaved RoPE,
  NHD/HND cache views, static per-tensor/per-head FP8 scales):
  rope_style="interleaved" rotates adjacent pairs (rope.rope_interleaved_*);
  layout="hnd" stores the pools as [num_blocks][Hkv][block_size][D] (FP4:
  codes [Hkv][block_size][D/2], then scales [Hkv][block_size][D/32] per
  block); a scale array of one element is a per-tensor scale, used for every
  kv head.

Storage arrays: act 'f32' -> float32 values, 'bf16' -> uint16 bits;
cache 'f32' -> float32, 'bf16' -> uint16 bits, 'fp8' -> uint8 codes,
'fp4' -> uint8 blocks [num_blocks, block_bytes] (codes, then scales).

Two modes:
  mode="recipe"  the fp32 evaluation recipe (rope.rope_f32_recipe, fp32
                 division by the scale) then rounding to storage: this is what
                 must match the device bit for bit;
  mode="exact"   the fp64 rotation rounded once to storage (the mathematical
                 result), for the within-one-ulp check.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import codecs, rope


def act_to_f64(x, act: str) -> np.ndarray:
    if act == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if act == "bf16":
        return codecs.bf16_decode(x)
    raise ValueError(act)


def f64_to_act(y, act: str) -> np.ndarray:
    """Round once to the activation storage dtype."""
    if act == "f32":
        return np.asarray(y, dtype=np.float64).astype(np.float32)
    if act == "bf16":
        return codecs.bf16_encode(y)
    raise ValueError(act)


def f64_to_cache(y, cache: str, scale: Optional[np.ndarray], fp32_div: bool) -> np.ndarray:
    """Round once to cache storage; FP8 divides by the per-head scale first
    (axis -2 is the kv head).  fp32_div selects an fp32 division (recipe)."""
    if cache == "f32":
        return np.asarray(y, dtype=np.float64).astype(np.float32)
    if cache == "bf16":
        return codecs.bf16_encode(y)
    if cache == "fp8":
        s = np.asarray(scale, dtype=np.float32)[:, None]
        if fp32_div:
            q = np.divide(np.asarray(y, dtype=np.float32), s, dtype=np.float32).astype(np.float64)
        else:
            q = np.asarray(y, dtype=np.float64) / s.astype(np.float64)
        return codecs.e4m3_encode(q)
    raise ValueError(cache)


@dataclass
class AppendResult:
    q_out: np.ndarray        # [B, Hq, D] act storage
    k_pool: np.ndarray       # updated copies of the pools (cache storage)
    v_pool: np.ndarray
    q_rot: np.ndarray        # [B, Hq, D] rotated Q before rounding (float64 of the mode's values)
    k_rot: np.ndarray        # [B, Hkv, D] rotated K before rounding
    v_new: np.ndarray        # [B, Hkv, D] V before rounding
    slots: list              # per sequence: (physical block, slot) written, or None


def pool_view(pool, cache: str, block_size: int, num_kv_heads: int, head_dim: int, layout: str = "nhd"):
    """A pool as [NB, block_size, Hkv, ...] views (for FP4 the pair (codes,
    scales)); for HND the block and head axes of the stored array are swapped,
    so writes through the view land in the stored layout."""
    p = np.asarray(pool)
    if cache == "fp4":
        return codecs.fp4_block_views(p, block_size, num_kv_heads, head_dim, layout)
    if layout == "hnd":
        return np.swapaxes(p, 1, 2)
    if layout != "nhd":
        raise ValueError(layout)
    return p


def rope_kv_append(qkv, context_lens, block_tables, k_pool, v_pool, *, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, block_size: int, act: str, cache: str,
                   rope_theta: float, k_scale=None, v_scale=None, mode: str = "recipe",
                   rope_style: str = "neox", layout: str = "nhd") -> AppendResult:
    Hq, Hkv, D, bs = num_q_heads, num_kv_heads, head_dim, block_size
    qkv = np.asarray(qkv)
    B = qkv.shape[0]
    ctx = np.asarray(context_lens, dtype=np.int64)
    x = act_to_f64(qkv[:, : (Hq + 2 * Hkv) * D], act).reshape(B, Hq + 2 * Hkv, D)
    pos = np.where(ctx >= 1, ctx - 1, 0)

    q_in, k_in, v_in = x[:, :Hq], x[:, Hq:Hq + Hkv], x[:, Hq + Hkv:]
    if mode == "recipe":
        q_rot = rope.rope_f32_recipe(q_in.astype(np.float32), pos, rope_theta, rope_style).astype(np.float64)
        k_rot = rope.rope_f32_recipe(k_in.astype(np.float32), pos, rope_theta, rope_style).astype(np.float64)
    elif mode == "exact":
        q_rot = rope.rope_f64(q_in, pos, rope_theta, rope_style)
        k_rot = rope.rope_f64(k_in, pos, rope_theta, rope_style)
    else:
        raise ValueError(mode)

    q_out = f64_to_act(q_rot, act)
    k_new = np.array(k_pool, copy=True)
    v_new_pool = np.array(v_pool, copy=True)
    kview = pool_view(k_new, cache, bs, Hkv, D, layout)
    vview = pool_view(v_new_pool, cache, bs, Hkv, D, layout)
    if cache == "fp4":
        k_parts, v_parts = kview, vview
        assert all(np.shares_memory(a, base) for a, base in ((k_parts[0], k_new), (v_parts[1], v_new_pool)))
    else:
        assert np.shares_memory(kview, k_new) and np.shares_memory(vview, v_new_pool)
    slots = []
    bt = np.asarray(block_tables)
    for b in range(B):
        if ctx[b] <= 0:
            slots.append(None)
            continue
        p = int(ctx[b] - 1)
        pb, off = int(bt[b, p // bs]), p % bs
        if cache == "fp4":
            for parts, rows in ((k_parts, k_rot[b]), (v_parts, v_in[b])):
                codes, scale_bytes = codecs.mx_fp4_quantize(rows)
                parts[0][pb, off] = codecs.fp4_pack(codes)
                parts[1][pb, off] = scale_bytes
        else:
            kview[pb, off] = f64_to_cache(k_rot[b], cache, k_scale, fp32_div=(mode == "recipe"))
            vview[pb, off] = f64_to_cache(v_in[b], cache, v_scale, fp32_div=(mode == "recipe"))
        slots.append((pb, off))
    return AppendResult(q_out, k_new, v_new_pool, q_rot, k_rot, v_in, slots)
