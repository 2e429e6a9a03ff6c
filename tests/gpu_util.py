"""Helpers for the GPU parity tests: move a seeded workload to the device, run
the library through the C ABI, and compute the oracle's expectation from the
same host inputs (never from anything the library produced)."""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import workloads as W
from oracle import append as OAP
from oracle import attention as OA
from oracle import codecs
from paged_gqa_decode_lgm_amd import ops

TOL = {"f32": 1e-5, "bf16": 2e-2}   # max-abs on attention outputs, by activation dtype


def announce(*parts):
    print("[gpu]", *parts, file=sys.stderr, flush=True)


@dataclasses.dataclass
class Dev:
    w: W.Workload
    qkv: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]

    @property
    def cfg(self):
        return self.w.cfg

    @property
    def max_ctx(self) -> int:
        return int(self.w.context_lens.max().item()) if self.w.cfg.num_seqs else 0


def to_device(w: W.Workload) -> Dev:
    cu = lambda t: None if t is None else t.to("cuda")
    c = w.cfg
    if c.cache == "fp4":
        pool = lambda t: ops.FP4Pool(t.to("cuda"), c.block_size, c.num_kv_heads, c.head_dim)
    else:
        pool = cu
    return Dev(w, cu(w.qkv), pool(w.k_pool), pool(w.v_pool), cu(w.block_tables), cu(w.context_lens),
               cu(w.k_scale), cu(w.v_scale))


def gpu_append(d: Dev) -> torch.Tensor:
    c = d.cfg
    return ops.rope_kv_append(d.qkv, d.k_pool, d.v_pool, d.block_tables, d.context_lens, c.rope_theta,
                              c.num_q_heads, d.k_scale, d.v_scale, layout=c.cache_layout, rope_style=c.rope_style)


def gpu_attention(d: Dev, q: torch.Tensor, partition_size: Optional[int] = None, max_ctx: Optional[int] = None):
    c = d.cfg
    ps = c.partition_size if partition_size is None else partition_size
    mc = d.max_ctx if max_ctx is None else max_ctx
    return ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                                 softmax_scale=c.softmax_scale, partition_size=ps,
                                 k_scale=d.k_scale, v_scale=d.v_scale, layout=c.cache_layout)


# ------------------------------------------------------------------ host views
def host_bits(t: torch.Tensor) -> np.ndarray:
    return W.storage_bits(t.detach().cpu())


def pool_raw(w: W.Workload, pool: torch.Tensor) -> np.ndarray:
    """Oracle's view of a cache pool: float32 values or raw storage bits."""
    return pool.numpy() if w.cfg.cache == "f32" else W.storage_bits(pool)


def act_raw(w: W.Workload, t: torch.Tensor) -> np.ndarray:
    return t.numpy() if w.cfg.act == "f32" else W.storage_bits(t)


def act_values(cfg, raw) -> np.ndarray:
    return OAP.act_to_f64(raw, cfg.act)


def oracle_append(w: W.Workload, mode: str):
    c = w.cfg
    return OAP.rope_kv_append(
        act_raw(w, w.qkv), w.context_lens.numpy(), w.block_tables.numpy(), pool_raw(w, w.k_pool),
        pool_raw(w, w.v_pool), num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
        block_size=c.block_size, act=c.act, cache=c.cache, rope_theta=c.rope_theta,
        k_scale=None if w.k_scale is None else w.k_scale.numpy(),
        v_scale=None if w.v_scale is None else w.v_scale.numpy(), mode=mode, rope_style=c.rope_style,
        layout=c.cache_layout)


def oracle_attention(w: W.Workload, q_raw: np.ndarray, k_pool_raw, v_pool_raw, seqs=None, ctx=None):
    c = w.cfg
    q = act_values(c, q_raw)
    return OA.paged_decode(q, k_pool_raw, v_pool_raw, w.block_tables.numpy(),
                           w.context_lens.numpy() if ctx is None else ctx, c.softmax_scale,
                           num_kv_heads=c.num_kv_heads, block_size=c.block_size, cache=c.cache,
                           k_scale=None if w.k_scale is None else w.k_scale.numpy(),
                           v_scale=None if w.v_scale is None else w.v_scale.numpy(), seqs=seqs,
                           layout=c.cache_layout)


def q_from_qkv(w: W.Workload) -> torch.Tensor:
    """Attention-only workloads use the Q part of the packed rows as q."""
    c = w.cfg
    return w.qkv[:, : c.num_q_heads * c.head_dim].reshape(c.num_seqs, c.num_q_heads, c.head_dim).contiguous()


# ------------------------------------------------------------------ comparisons
def bf16_ord(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def out_values(cfg, t: torch.Tensor) -> np.ndarray:
    return act_values(cfg, act_raw_tensor(cfg, t))


def act_raw_tensor(cfg, t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    return t.numpy() if cfg.act == "f32" else W.storage_bits(t)


def max_abs(a, b, rows=None) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if rows is not None:
        a, b = a[rows], b[rows]
    return float(np.abs(a - b).max()) if a.size else 0.0
