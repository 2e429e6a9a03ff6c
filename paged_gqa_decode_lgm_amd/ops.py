"""Torch-tensor front end of the C ABI: infers lgm_paged_dims from tensor
shapes, maps torch dtypes to lgm_dtype and allocates outputs / workspace with
torch (device memory is torch's job).  Every step of the decode path runs in
liblgm.so; nothing here computes any of it.

Shapes: qkv [B, (Hq+2Hkv)*D], q [B, Hq, D] (rows may be strided), caches
[num_blocks, block_size, Hkv, D] (NHD) or FP4Pool, block_tables int32
[B, MB], context_lens int32 [B].
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _binding as B

_DTYPES = {torch.float32: B.LGM_F32, torch.bfloat16: B.LGM_BF16, torch.float8_e4m3fn: B.LGM_FP8_E4M3}


class FP4Pool:
    """An FP4 cache pool (LGM_FP4_E2M1): ``data`` is uint8 [num_blocks,
    block_bytes], each block its NHD E2M1 codes [block_size][Hkv][D/2] (two
    per byte, low nibble first) followed by its E8M0 scales
    [block_size][Hkv][D/32].  ``shape`` is the logical (num_blocks,
    block_size, Hkv, D)."""

    def __init__(self, data: torch.Tensor, block_size: int, num_kv_heads: int, head_dim: int):
        if head_dim % 32:
            raise ValueError("FP4 pools need head_dim a multiple of 32")
        nbytes = block_size * num_kv_heads * (head_dim // 2 + head_dim // 32)
        if data.dtype != torch.uint8 or data.dim() != 2 or data.shape[1] != nbytes or not data.is_contiguous():
            raise ValueError(f"FP4 pool data must be contiguous uint8 [num_blocks, {nbytes}]")
        self.data = data
        self.shape = (data.shape[0], block_size, num_kv_heads, head_dim)

    @property
    def device(self):
        return self.data.device

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def lgm_dtype(t) -> int:
    if isinstance(t, FP4Pool):
        return B.LGM_FP4_E2M1
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"no lgm_dtype for {t.dtype}") from None


def dims_for(num_seqs: int, num_q_heads: int, k_cache, block_tables: torch.Tensor,
             layout: str = "nhd") -> B.lgm_paged_dims:
    """Dims from a cache's shape: [NB, bs, Hkv, D] (NHD), [NB, Hkv, bs, D]
    (HND tensors) or an FP4Pool's logical shape (always (NB, bs, Hkv, D))."""
    if layout == "hnd" and not isinstance(k_cache, FP4Pool):
        nb, hkv, bs, d = k_cache.shape
    else:
        nb, bs, hkv, d = k_cache.shape
    return B.make_dims(num_seqs, num_q_heads, hkv, d, bs, nb, block_tables.shape[1])


def variant_flags(layout: str = "nhd", rope_style: str = "neox", k_scale=None, num_kv_heads: int = 1) -> int:
    """lgm flags for a cache layout ("nhd" / "hnd"), a RoPE style ("neox" /
    "interleaved") and FP8 scales given as one value for all kv heads."""
    if layout not in ("nhd", "hnd") or rope_style not in ("neox", "interleaved"):
        raise ValueError(f"layout {layout!r} / rope_style {rope_style!r}")
    f = B.LGM_CACHE_HND if layout == "hnd" else 0
    f |= B.LGM_ROPE_INTERLEAVED if rope_style == "interleaved" else 0
    if k_scale is not None and k_scale.numel() == 1 and num_kv_heads > 1:
        f |= B.LGM_SCALE_PER_TENSOR
    return f


def rope_kv_append(qkv, k_cache, v_cache, block_tables, context_lens, rope_theta: float, num_q_heads: int,
                   k_scale=None, v_scale=None, q_out=None, stream=None, layout: str = "nhd",
                   rope_style: str = "neox") -> torch.Tensor:
    """Rotate Q/K of the new token, append K/V into the paged caches; returns q_out [B, Hq, D]."""
    bsz = qkv.shape[0]
    d = k_cache.shape[3]
    if q_out is None:
        q_out = torch.empty((bsz, num_q_heads, d), dtype=qkv.dtype, device=qkv.device)
    dims = dims_for(bsz, num_q_heads, k_cache, block_tables, layout)
    flags = variant_flags(layout, rope_style, k_scale, dims.num_kv_heads)
    B.lgm_rope_kv_append(qkv, qkv.stride(0), q_out, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                         float(rope_theta), dims, lgm_dtype(qkv), lgm_dtype(k_cache), flags=flags, stream=stream)
    return q_out


def workspace_bytes(q, k_cache, block_tables, max_context_len: int, partition_size: int = 0,
                    layout: str = "nhd") -> int:
    dims = dims_for(q.shape[0], q.shape[1], k_cache, block_tables, layout)
    return B.lgm_paged_decode_workspace_size(dims, max_context_len, partition_size, lgm_dtype(k_cache))


def partition_size(q, k_cache, block_tables, max_context_len: int, partition_size: int = 0,
                   layout: str = "nhd") -> int:
    dims = dims_for(q.shape[0], q.shape[1], k_cache, block_tables, layout)
    return B.lgm_paged_decode_partition_size(dims, max_context_len, partition_size, lgm_dtype(k_cache))


def paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                      softmax_scale: Optional[float] = None, partition_size: int = 0, k_scale=None, v_scale=None,
                      out=None, out_lse=None, workspace=None, want_lse: bool = True,
                      stream=None, layout: str = "nhd") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode attention of q [B, Hq, D] over the paged caches; returns (out, lse)."""
    bsz, hq, d = q.shape
    if q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError("q must be [B, Hq, D] with heads dense (only the sequence stride may differ)")
    dims = dims_for(bsz, hq, k_cache, block_tables, layout)
    flags = variant_flags(layout, "neox", k_scale, dims.num_kv_heads)
    if softmax_scale is None:
        softmax_scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((bsz, hq, d), dtype=q.dtype, device=q.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    need = B.lgm_paged_decode_workspace_size(dims, max_context_len, partition_size, lgm_dtype(k_cache))
    if workspace is None and need:
        # zero-filled: the matrix-core kernel keeps its work counters at its start
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    B.lgm_paged_decode_attn(out, out_lse, q, q.stride(0), k_cache, v_cache, block_tables, context_lens, k_scale,
                            v_scale, float(softmax_scale), partition_size, int(max_context_len), workspace, ws_bytes,
                            dims, lgm_dtype(q), lgm_dtype(k_cache), flags=flags, stream=stream)
    return out, out_lse


def paged_decode_attn_static(q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                             softmax_scale: Optional[float] = None, partition_size: int = 0, k_scale=None,
                             v_scale=None, out=None, out_lse=None, want_lse: bool = True, stream=None,
                             layout: str = "nhd") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """paged_decode_attn on the library's device-resident scratch array
    (lgm_paged_decode_attn_static): no workspace is passed or allocated."""
    bsz, hq, d = q.shape
    if q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError("q must be [B, Hq, D] with heads dense (only the sequence stride may differ)")
    dims = dims_for(bsz, hq, k_cache, block_tables, layout)
    flags = variant_flags(layout, "neox", k_scale, dims.num_kv_heads)
    if softmax_scale is None:
        softmax_scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((bsz, hq, d), dtype=q.dtype, device=q.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    B.lgm_paged_decode_attn_static(out, out_lse, q, q.stride(0), k_cache, v_cache, block_tables, context_lens,
                                   k_scale, v_scale, float(softmax_scale), partition_size, int(max_context_len), dims,
                                   lgm_dtype(q), lgm_dtype(k_cache), flags=flags, stream=stream)
    return out, out_lse


def check_block_tables(k_cache, block_tables, context_lens, max_context_len: int, status=None, stream=None,
                       layout: str = "nhd") -> torch.Tensor:
    """Enqueues lgm_check_block_tables; returns its int32 [4] status words
    (zero-filled here when not given; read them after synchronising)."""
    dims = dims_for(block_tables.shape[0], 1, k_cache, block_tables, layout)
    dims.num_q_heads = dims.num_kv_heads  # the check reads no query
    if status is None:
        status = torch.zeros(4, dtype=torch.int32, device=block_tables.device)
    B.lgm_check_block_tables(block_tables, context_lens, dims, int(max_context_len), status, stream)
    return status


def lse_merge(partial_out, partial_lse, num_partitions=None, out_dtype=torch.float32, out=None, out_lse=None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge records partial_out [B, H, P, D] / partial_lse [B, H, P]."""
    bsz, h, p, d = partial_out.shape
    if out is None:
        out = torch.empty((bsz, h, d), dtype=out_dtype, device=partial_out.device)
    if out_lse is None:
        out_lse = torch.empty((bsz, h), dtype=torch.float32, device=partial_out.device)
    B.lgm_lse_merge(out, out_lse, partial_out, partial_lse, num_partitions, bsz, h, d, p, lgm_dtype(out), stream)
    return out, out_lse


# ---- paged MLA (include/lgm_mla.h) -----------------------------------------------------
def mla_dims_for(q_latent, q_pe, ckv_cache, block_tables) -> B.lgm_mla_dims:
    """Dims from q_latent [B, H, 512], q_pe [B, H, 64], ckv [NB, bs, 512]."""
    bsz, h, dl = q_latent.shape
    nb, bs, _ = ckv_cache.shape
    return B.make_mla_dims(bsz, h, dl, q_pe.shape[2], bs, nb, block_tables.shape[1])


def mla_partition_size(q_latent, q_pe, ckv_cache, block_tables, max_context_len: int, partition_size: int = 0) -> int:
    dims = mla_dims_for(q_latent, q_pe, ckv_cache, block_tables)
    return B.lgm_paged_mla_partition_size(dims, int(max_context_len), partition_size)


def mla_workspace_bytes(q_latent, q_pe, ckv_cache, block_tables, max_context_len: int,
                        partition_size: int = 0) -> int:
    dims = mla_dims_for(q_latent, q_pe, ckv_cache, block_tables)
    return B.lgm_paged_mla_workspace_size(dims, int(max_context_len), partition_size)


def paged_mla_decode(q_latent, q_pe, ckv_cache, kpe_cache, block_tables, context_lens, max_context_len: int,
                     softmax_scale: float, ckv_scale, partition_size: int = 0, out=None, out_lse=None,
                     workspace=None, want_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged MLA decode of q_latent [B, H, 512] / q_pe [B, H, 64] (bf16,
    dense) over ckv [NB, bs, 512] (float8_e4m3fn) and kpe [NB, bs, 64]
    (bf16); returns (out [B, H, 512] bf16, lse [B, H] or None)."""
    for name, t in (("q_latent", q_latent), ("q_pe", q_pe), ("ckv_cache", ckv_cache), ("kpe_cache", kpe_cache)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dims = mla_dims_for(q_latent, q_pe, ckv_cache, block_tables)
    bsz, h, dl = q_latent.shape
    if out is None:
        out = torch.empty((bsz, h, dl), dtype=torch.bfloat16, device=q_latent.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((bsz, h), dtype=torch.float32, device=q_latent.device)
    need = B.lgm_paged_mla_workspace_size(dims, int(max_context_len), partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_latent.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    B.lgm_paged_mla_decode(out, out_lse, q_latent, q_pe, ckv_cache, kpe_cache, block_tables, context_lens, ckv_scale,
                           float(softmax_scale), partition_size, int(max_context_len), workspace, ws_bytes, dims,
                           lgm_dtype(ckv_cache), stream=stream)
    return out, out_lse
