"""Paged GQA/MQA single-token decode attention, split-K partials and their
log-sum-exp merge (oracle only, fp64).

The method on the pages (mainarch README, decode-attention section: one
query over a long KV cache, FlashDecoding split-KV with online softmax and a
combine of the partial results, paged KV through a block table, GQA reading
each KV head once for its query-head group; Loom Kernels, "Supported operator
paths": paged MQA/GQA decode with GQA reuse and a local split-K/LSE merge)
reaches exactly, up to rounding order, plain softmax attention over the
gathered cache.  So the oracle is that definition written out; it does not
reproduce online softmax or any tiling.

For sequence b, query head h with kv head g = h // G (contiguous groups of
G = Hq / Hkv query heads; the pages only say that a group of query heads
shares one KV head) and L = context_lens[b]:
    K_j, V_j = cache rows of token j < L, found through the block table:
               physical block block_tables[b, j // bs], slot j % bs
               (FP8 rows are decoded and multiplied by the head's scale, or
               the single per-tensor scale;
               FP4 rows are E2M1 codes times their 32-element blocks' E8M0
               scales, oracle.codecs)
    s_j   = scale * <q_h, K_j>
    p     = softmax(s)
    out_h = sum_j p_j V_j,   lse_h = log sum_j exp(s_j)   (natural log)
L = 0 gives out = 0 and lse = -inf.  The pools are NHD ([NB][bs][Hkv][D]) or,
with layout="hnd", [NB][Hkv][bs][D] (Loom's "NHD/HND cache views").

Split-K (the reading taken of "split-K partitions merged by log-sum-exp"):
partition p covers tokens [p*PS, min((p+1)*PS, L)), P_b = ceil(L / PS);
each partition's record is its own normalised softmax output o_p and its
log-sum-exp lse_p; the merge is
    M = max_p lse_p,  w_p = exp(lse_p - M),
    out = sum_p w_p o_p / sum_p w_p,  lse = M + log sum_p w_p.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import codecs


def decode_rows(raw, cache: str, scale_g: Optional[float] = None) -> np.ndarray:
    """Cache storage -> float64 values (FP8: decoded byte times the scale;
    FP4: raw is (packed codes, scale bytes) of the rows)."""
    if cache == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if cache == "bf16":
        return codecs.bf16_decode(raw)
    if cache == "fp8":
        return codecs.e4m3_decode(raw) * np.float64(np.float32(scale_g))
    if cache == "fp4":
        return codecs.mx_fp4_dequantize(*raw)
    raise ValueError(cache)


def kv_source(pool, cache: str, block_size: int, num_kv_heads: int, head_dim: int, layout: str = "nhd"):
    """A pool as gather_kv indexes it: [NB, bs, Hkv, D] storage, or for FP4
    (uint8 [NB, block_bytes] blocks of codes then scales) the pair of views
    (codes [NB, bs, Hkv, D/2], scales [NB, bs, Hkv, D/32]).  An HND pool
    ([NB, Hkv, bs, D]; FP4: each part head-major) is viewed with the block
    and head axes swapped, so the gather is the same for both layouts."""
    if cache == "fp4":
        return codecs.fp4_block_views(pool, block_size, num_kv_heads, head_dim, layout)
    p = np.asarray(pool)
    if layout == "hnd":
        return np.swapaxes(p, 1, 2)
    if layout != "nhd":
        raise ValueError(layout)
    return p


def gather_kv(pool, block_tables, b: int, L: int, g: int, block_size: int, cache: str,
              scale=None) -> np.ndarray:
    """Rows j < L of kv head g for sequence b, through the block table: [L, D].
    ``pool`` as kv_source returns it."""
    if L <= 0:
        D = 2 * pool[0].shape[-1] if cache == "fp4" else pool.shape[-1]
        return np.zeros((0, D), dtype=np.float64)
    j = np.arange(L)
    pb = np.asarray(block_tables)[b, j // block_size].astype(np.int64)
    if cache == "fp4":
        codes, scales = pool
        return decode_rows((codes[pb, j % block_size, g, :], scales[pb, j % block_size, g, :]), cache)
    raw = np.asarray(pool)[pb, j % block_size, g, :]
    sc = None if scale is None else np.asarray(scale).reshape(-1)
    sg = None if sc is None else float(sc[g] if sc.size > 1 else sc[0])  # one element: a per-tensor scale
    return decode_rows(raw, cache, sg)


def attend(q, K, V, scale: float):
    """Softmax attention of query rows q [n, D] over K, V [L, D] (fp64).
    Returns (out [n, D], lse [n], p [n, L])."""
    q = np.asarray(q, dtype=np.float64)
    n, D = q.shape
    L = K.shape[0]
    if L == 0:
        return np.zeros((n, D)), np.full(n, -np.inf), np.zeros((n, 0))
    s = np.float64(scale) * (q @ K.T)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    p = w / l
    return p @ V, (m + np.log(l))[:, 0], p


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, softmax_scale: float, *,
                 num_kv_heads: int, block_size: int, cache: str, k_scale=None, v_scale=None,
                 seqs: Optional[Iterable[int]] = None, layout: str = "nhd"):
    """out [B, Hq, D] and lse [B, Hq] in fp64.  q: [B, Hq, D] (float64 values).
    ``seqs`` restricts the work to some sequences (others are NaN)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    ctx = np.asarray(context_lens, dtype=np.int64)
    k_pool = kv_source(k_pool, cache, block_size, num_kv_heads, D, layout)
    v_pool = kv_source(v_pool, cache, block_size, num_kv_heads, D, layout)
    for b in (range(B) if seqs is None else seqs):
        L = max(int(ctx[b]), 0)
        for g in range(num_kv_heads):
            K = gather_kv(k_pool, block_tables, b, L, g, block_size, cache, k_scale)
            V = gather_kv(v_pool, block_tables, b, L, g, block_size, cache, v_scale)
            o, ls, _ = attend(q[b, g * G:(g + 1) * G], K, V, softmax_scale)
            out[b, g * G:(g + 1) * G] = o
            lse[b, g * G:(g + 1) * G] = ls
    return out, lse


def num_partitions(context_lens, partition_size: int) -> np.ndarray:
    ctx = np.maximum(np.asarray(context_lens, dtype=np.int64), 0)
    return -(-ctx // partition_size)


def paged_decode_partials(q, k_pool, v_pool, block_tables, context_lens, softmax_scale: float,
                          partition_size: int, *, num_kv_heads: int, block_size: int, cache: str,
                          k_scale=None, v_scale=None, layout: str = "nhd"):
    """Per-partition records: o_p [B, Hq, Pmax, D] (normalised), lse_p
    [B, Hq, Pmax] and P_b [B].  Records at p >= P_b are zeros / -inf."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    PS = int(partition_size)
    nparts = num_partitions(context_lens, PS)
    Pmax = max(int(nparts.max()) if B else 0, 1)
    o_p = np.zeros((B, Hq, Pmax, D))
    lse_p = np.full((B, Hq, Pmax), -np.inf)
    ctx = np.asarray(context_lens, dtype=np.int64)
    k_pool = kv_source(k_pool, cache, block_size, num_kv_heads, D, layout)
    v_pool = kv_source(v_pool, cache, block_size, num_kv_heads, D, layout)
    for b in range(B):
        L = max(int(ctx[b]), 0)
        for g in range(num_kv_heads):
            K = gather_kv(k_pool, block_tables, b, L, g, block_size, cache, k_scale)
            V = gather_kv(v_pool, block_tables, b, L, g, block_size, cache, v_scale)
            for p in range(int(nparts[b])):
                lo, hi = p * PS, min((p + 1) * PS, L)
                o, ls, _ = attend(q[b, g * G:(g + 1) * G], K[lo:hi], V[lo:hi], softmax_scale)
                o_p[b, g * G:(g + 1) * G, p] = o
                lse_p[b, g * G:(g + 1) * G, p] = ls
    return o_p, lse_p, nparts


def lse_merge(o_p, lse_p, num_parts=None):
    """Merge partition records [B, H, P, D] / [B, H, P] by log-sum-exp.
    ``num_parts`` [B] limits each sequence to its first P_b records.

    A record whose lse is -inf is an empty partition (its softmax sums over
    no token): it is left out of the merge altogether, so whatever its
    output row holds (zeros, or NaN/Inf in memory nobody wrote) has no
    effect.  That is the reading taken of "an empty partition weighs zero"
    (the combine of split partials in the mainarch README's decode-attention
    section; the local split-K/LSE merge of the Loom Kernels README, row
    "Attention"): its weight exp(-inf) is exactly 0, and 0 times its row is
    taken as 0 even where IEEE arithmetic would give NaN."""
    o_p = np.asarray(o_p, dtype=np.float64)
    lse_p = np.asarray(lse_p, dtype=np.float64)
    B, H, P, D = o_p.shape
    out = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = P if num_parts is None else int(num_parts[b])
        for h in range(H):
            ls = lse_p[b, h, :n]
            live = ls > -np.inf
            if not live.any():
                continue
            ls = ls[live]
            M = ls.max()
            w = np.exp(ls - M)
            out[b, h] = (w[:, None] * o_p[b, h, :n][live]).sum(axis=0) / w.sum()
            lse[b, h] = M + np.log(w.sum())
    return out, lse
