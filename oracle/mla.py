"""Paged multi-head latent attention (MLA) decode (oracle only, fp64).

mainarch's decode-attention section describes the latent path: the cache
holds, per token, a 512-dimensional compressed latent (FP8 E4M3 "ckv") and a
64-dimensional positional part (bf16 "kpe") instead of per-head K and V; the
per-head projections happen after the cache read, so every query head
attends to the same latent rows.  Its kernel computes per-head dot scores,
a local softmax with exported LSE and softmax-weighted latent output tiles,
split-K across the sequence with a stage-2 merge of the partial records.

Readings (the pages give no formula):
* query head h brings a latent query q_lat[h] (512) and a positional query
  q_pe[h] (64), i.e. the absorbed form; the score of token j is
      s_j = scale * (<q_lat[h], c_j> + <q_pe[h], r_j>)
  with c_j = decode(ckv_j) * ckv_scale (a static per-tensor FP8 scale) and
  r_j = kpe_j;
* the value of token j is its latent c_j, so out[h] = sum_j softmax(s)_j c_j
  (512-dimensional, natural-log LSE as for the GQA path);
* the cache is paged like the GQA pools: ckv [num_blocks][block_size][512]
  and kpe [num_blocks][block_size][64], one block table for both;
* split-K partitions and their merge are those of oracle.attention (the
  same log-sum-exp combine).

This is the plain definition: the gathered rows, the dot products, a softmax
and a weighted sum, in fp64.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import codecs


def gather_latent(ckv_pool, kpe_pool, block_tables, b: int, L: int, block_size: int, ckv_cache: str,
                  ckv_scale: float):
    """Latent rows c [L, 512] and positional rows r [L, 64] of sequence b (fp64)."""
    if L <= 0:
        return np.zeros((0, np.asarray(ckv_pool).shape[-1])), np.zeros((0, np.asarray(kpe_pool).shape[-1]))
    j = np.arange(L)
    pb = np.asarray(block_tables)[b, j // block_size].astype(np.int64)
    craw = np.asarray(ckv_pool)[pb, j % block_size]
    rraw = np.asarray(kpe_pool)[pb, j % block_size]
    if ckv_cache == "fp8":
        c = codecs.e4m3_decode(craw) * np.float64(np.float32(ckv_scale))
    elif ckv_cache == "bf16":
        c = codecs.bf16_decode(craw)
    else:
        raise ValueError(ckv_cache)
    return c, codecs.bf16_decode(rraw)


def mla_attend(q_lat, q_pe, c, r, scale: float):
    """Attention of query heads (q_lat [H, 512], q_pe [H, 64]) over latent rows
    c [L, 512] and positional rows r [L, 64].  Returns (out [H, 512], lse [H])."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    H = q_lat.shape[0]
    if c.shape[0] == 0:
        return np.zeros((H, c.shape[1])), np.full(H, -np.inf)
    s = np.float64(scale) * (q_lat @ c.T + q_pe @ r.T)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    return (w / l) @ c, (m + np.log(l))[:, 0]


def paged_mla_decode(q_lat, q_pe, ckv_pool, kpe_pool, block_tables, context_lens, softmax_scale: float, *,
                     block_size: int, ckv_cache: str = "fp8", ckv_scale: float = 1.0,
                     seqs: Optional[Iterable[int]] = None):
    """out [B, H, 512] and lse [B, H] (fp64); q_lat [B, H, 512], q_pe [B, H, 64]
    as float64 values.  ``seqs`` restricts the work (others are NaN)."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, H, DL = q_lat.shape
    out = np.full((B, H, DL), np.nan)
    lse = np.full((B, H), np.nan)
    ctx = np.asarray(context_lens, dtype=np.int64)
    for b in (range(B) if seqs is None else seqs):
        c, r = gather_latent(ckv_pool, kpe_pool, block_tables, b, max(int(ctx[b]), 0), block_size, ckv_cache,
                             ckv_scale)
        out[b], lse[b] = mla_attend(q_lat[b], q_pe[b], c, r, softmax_scale)
    return out, lse


def paged_mla_partials(q_lat, q_pe, ckv_pool, kpe_pool, block_tables, context_lens, softmax_scale: float,
                       partition_size: int, *, block_size: int, ckv_cache: str = "fp8", ckv_scale: float = 1.0):
    """Split-K records: o_p [B, H, Pmax, 512], lse_p [B, H, Pmax] and P_b [B],
    partition p covering tokens [p*PS, min((p+1)*PS, L))."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, H, DL = q_lat.shape
    PS = int(partition_size)
    ctx = np.maximum(np.asarray(context_lens, dtype=np.int64), 0)
    nparts = -(-ctx // PS)
    Pmax = max(int(nparts.max()) if B else 0, 1)
    o_p = np.zeros((B, H, Pmax, DL))
    lse_p = np.full((B, H, Pmax), -np.inf)
    for b in range(B):
        L = int(ctx[b])
        c, r = gather_latent(ckv_pool, kpe_pool, block_tables, b, L, block_size, ckv_cache, ckv_scale)
        for p in range(int(nparts[b])):
            lo, hi = p * PS, min((p + 1) * PS, L)
            o_p[b, :, p], lse_p[b, :, p] = mla_attend(q_lat[b], q_pe[b], c[lo:hi], r[lo:hi], softmax_scale)
    return o_p, lse_p, nparts
