"""Seeded synthetic inputs for paged GQA/MQA decode attention.

This module only *draws inputs*: context lengths, block tables, cache pools,
packed QKV rows and static FP8 scales.  FP4 pools are drawn directly as
bytes (uniform E2M1 codes, E8M0 scale bytes spread over the binades that
N(0,1) blocks of 32 land in), since turning drawn values into FP4 would be
the method's own quantisation.  It holds none of the decode method's
arithmetic (no RoPE, no attention, no merge, no quantised append).  Casts of
the drawn N(0,1) values into the storage dtypes use torch's own conversions
(round-to-nearest-even), so neither the oracle nor the HIP library lends it
any code.  Both sides of every parity test take their inputs from here.

Shapes follow the paged-KV contract described on the pages: NHD cache blocks
``[num_blocks][block_size][num_kv_heads][head_dim]`` addressed through an
int32 block table ``[B, max_blocks_per_seq]`` (Loom Kernels, "Supported
operator paths", row "Position and KV"; mainarch README, decode-attention
section: logical-to-physical block map with a deliberately shuffled layout).

Draw order is fixed by stage: each stage owns one child of
``numpy.random.SeedSequence(seed)``; large arrays are filled in fixed-size
chunks, chunk ``i`` from grandchild ``i``, so the bytes do not depend on the
number of threads used to fill them.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Tuple, Union

import numpy as np
import torch

# Stage indices of the draw order.
STAGE_CTX, STAGE_TABLE, STAGE_K, STAGE_V, STAGE_QKV, STAGE_OUTLIER, STAGE_CALIB = range(7)
_CHUNK = 1 << 22  # values per RNG chunk

DTYPE_F32, DTYPE_BF16, DTYPE_FP8, DTYPE_FP4 = "f32", "bf16", "fp8", "fp4"
ELEM_BYTES = {DTYPE_F32: 4, DTYPE_BF16: 2, DTYPE_FP8: 1}
FP4_SCALE_BLOCK = 32              # elements per E8M0 scale
FP4_SCALE_BYTES = (125, 126)  # drawn scale bytes 2**-2, 2**-1: |values| <= 3, rms ~1.2
TORCH_STORAGE = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16, DTYPE_FP8: torch.float8_e4m3fn}
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Config:
    """One decode workload.  ``ctx`` is a fixed length or an inclusive (lo, hi)."""

    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    act: str
    cache: str
    ctx: Union[int, Tuple[int, int]]
    rope_theta: float
    partition_size: int  # 0 = library chooses; >= max context = no split
    append: bool = True
    num_blocks: Optional[int] = None  # None = ceil(1.25 * blocks in use)
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    calib_tokens: int = 4096
    ctx_list: Optional[Tuple[int, ...]] = None  # explicit per-sequence lengths (overrides ctx)
    description: str = ""
    # contract variants (Loom's "Position and KV" row)
    rope_style: str = "neox"        # or "interleaved" (adjacent pairs)
    cache_layout: str = "nhd"       # or "hnd": [num_blocks][Hkv][block_size][D]
    scale_per_tensor: bool = False  # FP8: one K and one V scale for all kv heads

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_ctx(self) -> int:
        if self.ctx_list is not None:
            return max(self.ctx_list) if self.ctx_list else 0
        return self.ctx if isinstance(self.ctx, int) else self.ctx[1]

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_ctx // self.block_size)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads.  Shapes stand in for the models the pages discuss; no
# weights or datasets are involved.
CONFIGS = {
    "tiny_mqa_f32": Config(
        "tiny_mqa_f32", seed=1, num_seqs=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
        block_size=16, act=DTYPE_F32, cache=DTYPE_F32, ctx=256, rope_theta=1e4,
        partition_size=256, num_blocks=16,
        description="fp32 MQA 4/1, D64, ctx 256, bs16, permuted pool of 16 blocks, no split-K"),
    "qwen2.5_1.5b_gqa": Config(
        "qwen2.5_1.5b_gqa", seed=2, num_seqs=2, num_q_heads=12, num_kv_heads=2, head_dim=128,
        block_size=16, act=DTYPE_BF16, cache=DTYPE_BF16, ctx=2048, rope_theta=1e6,
        partition_size=0, num_blocks=4096,
        description="Qwen2.5-1.5B-shaped 12/2, D128, bf16, B2, ctx 2048, pool 4096 blocks"),
    "llama3_8b_gqa": Config(
        "llama3_8b_gqa", seed=3, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, act=DTYPE_BF16, cache=DTYPE_BF16, ctx=(512, 8192), rope_theta=5e5,
        partition_size=0,
        description="Llama-3-8B-shaped 32/8, D128, bf16, B64, ctx U[512,8192]"),
    "long_ctx_splitk": Config(
        "long_ctx_splitk", seed=4, num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, act=DTYPE_BF16, cache=DTYPE_BF16, ctx=131072, rope_theta=5e5,
        partition_size=512, append=False, outlier_frac=0.01, outlier_scale=8.0,
        description="32/8, D128, bf16, B4, ctx 131072, 512-token partitions, 1% K rows x8"),
    "fp8_kv": Config(
        "fp8_kv", seed=5, num_seqs=128, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, act=DTYPE_BF16, cache=DTYPE_FP8, ctx=(1024, 4096), rope_theta=5e5,
        partition_size=0,
        description="32/8, D128, FP8 E4M3 cache with static per-head scales, B128, ctx U[1024,4096]"),
    "fp4_kv": Config(
        "fp4_kv", seed=6, num_seqs=128, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, act=DTYPE_BF16, cache=DTYPE_FP4, ctx=(1024, 4096), rope_theta=5e5,
        partition_size=0,
        description="32/8, D128, FP4 E2M1 cache with E8M0 scales per 32 elements, B128, ctx U[1024,4096]"),
}


def fp4_block_bytes(block_size: int, num_kv_heads: int, head_dim: int) -> int:
    """Bytes of one FP4 cache block: NHD codes (two per byte), then one scale
    byte per 32 elements of each (token, kv head) row."""
    return block_size * num_kv_heads * (head_dim // 2 + head_dim // FP4_SCALE_BLOCK)


def row_bytes(cache: str, head_dim: int) -> int:
    """Bytes of one (token, kv head) row of a cache, scales included."""
    if cache == DTYPE_FP4:
        return head_dim // 2 + head_dim // FP4_SCALE_BLOCK
    return head_dim * ELEM_BYTES[cache]


@dataclasses.dataclass
class Workload:
    """Host-side inputs.  Storage tensors hold the exact bytes the GPU sees.

    k_pool / v_pool: [num_blocks, block_size, Hkv, D] in the cache storage dtype
    ([num_blocks, Hkv, block_size, D] for the HND layout; FP4: uint8
    [num_blocks, fp4_block_bytes], whose bytes are drawn uniformly, so the
    same draw serves either layout).
    qkv: [B, (Hq + 2*Hkv) * D] in the activation dtype; per row Q heads, then
    K heads, then V heads, each head_dim-contiguous.
    """

    cfg: Config
    context_lens: torch.Tensor  # int32 [B]
    block_tables: torch.Tensor  # int32 [B, MB]; unused entries are -1
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    qkv: torch.Tensor
    k_scale: Optional[torch.Tensor]  # fp32 [Hkv] for FP8 caches
    v_scale: Optional[torch.Tensor]

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one attention call reads: each (token, kv-head) row once."""
        c = self.cfg
        return int(self.context_lens.clamp(min=0).sum()) * 2 * c.num_kv_heads * row_bytes(c.cache, c.head_dim)


def _children(seed: int, stage: int, n: int):
    return np.random.SeedSequence([seed, stage]).spawn(n)


def _normal_f32(seed: int, stage: int, count: int, threads: int = 0) -> np.ndarray:
    """count N(0,1) float32 values, chunk i from its own grandchild seed."""
    out = np.empty(count, dtype=np.float32)
    nchunk = max(1, -(-count // _CHUNK))
    kids = _children(seed, stage, nchunk)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(count, (i + 1) * _CHUNK)
        np.random.default_rng(kids[i]).standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(nchunk)))
    return out


def draw_context_lens(cfg: Config) -> np.ndarray:
    if cfg.ctx_list is not None:
        if len(cfg.ctx_list) != cfg.num_seqs:
            raise ValueError("ctx_list needs one length per sequence")
        return np.asarray(cfg.ctx_list, dtype=np.int32)
    if isinstance(cfg.ctx, int):
        return np.full(cfg.num_seqs, cfg.ctx, dtype=np.int32)
    rng = np.random.default_rng(_children(cfg.seed, STAGE_CTX, 1)[0])
    lo, hi = cfg.ctx
    return rng.integers(lo, hi + 1, size=cfg.num_seqs, dtype=np.int64).astype(np.int32)


def draw_block_tables(cfg: Config, ctx: np.ndarray) -> Tuple[np.ndarray, int]:
    """Distinct physical blocks per sequence from a seeded permutation of the pool."""
    bs = cfg.block_size
    nblk = [-(-int(c) // bs) for c in ctx]
    used = sum(nblk)
    nb = cfg.num_blocks if cfg.num_blocks is not None else max(1, -(-used * 5 // 4))
    if used > nb:
        raise ValueError(f"{cfg.name}: pool of {nb} blocks cannot hold {used}")
    rng = np.random.default_rng(_children(cfg.seed, STAGE_TABLE, 1)[0])
    perm = rng.permutation(nb).astype(np.int32)
    mb = max(cfg.max_blocks_per_seq, max(nblk) if nblk else 1, 1)
    bt = np.full((cfg.num_seqs, mb), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, nb


def _to_storage(x_f32: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None) -> torch.Tensor:
    """Cast drawn fp32 values to storage with torch (RNE).  FP8 values are
    divided by their per-head scale (last-but-one axis = kv head) and clamped
    to the finite E4M3 range first."""
    t = torch.from_numpy(x_f32)
    if dtype == DTYPE_F32:
        return t.clone()
    if dtype == DTYPE_BF16:
        return t.to(torch.bfloat16)
    s = torch.from_numpy(scale.astype(np.float32)).view(-1, 1)
    return (t / s).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)


def draw_calibration_scales(cfg: Config) -> Tuple[np.ndarray, np.ndarray]:
    """Static FP8 scales: absmax / 448 of a seeded calibration draw of
    ``calib_tokens`` x D values per KV head, separately for K and V; per
    tensor, the absmax is taken over all heads and one scale is returned."""
    n = cfg.calib_tokens * cfg.head_dim
    x = _normal_f32(cfg.seed, STAGE_CALIB, 2 * cfg.num_kv_heads * n).reshape(2, cfg.num_kv_heads, n)
    amax = np.abs(x).max(axis=2).astype(np.float32)
    if cfg.scale_per_tensor:
        amax = amax.max(axis=1, keepdims=True)
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return scales[0].copy(), scales[1].copy()


def draw_fp4_pool(cfg: Config, stage: int, nb: int) -> torch.Tensor:
    """uint8 [nb, block_bytes]: each block's code bytes uniform over all 256
    (two uniform E2M1 codes), then its scale bytes uniform over FP4_SCALE_BYTES."""
    hkv, d, bs = cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    nc = bs * hkv * d // 2
    ns = bs * hkv * d // FP4_SCALE_BLOCK
    kid_codes, kid_scales = _children(cfg.seed, stage, 2)
    pool = np.empty((nb, nc + ns), dtype=np.uint8)
    pool[:, :nc] = np.random.default_rng(kid_codes).integers(0, 256, size=(nb, nc), dtype=np.uint8)
    choice = np.random.default_rng(kid_scales).integers(0, len(FP4_SCALE_BYTES), size=(nb, ns))
    pool[:, nc:] = np.asarray(FP4_SCALE_BYTES, dtype=np.uint8)[choice]
    return torch.from_numpy(pool)


def make_workload(cfg: Config) -> Workload:
    ctx = draw_context_lens(cfg)
    bt, nb = draw_block_tables(cfg, ctx)
    hkv, d, bs = cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    if cfg.cache == DTYPE_FP4:
        if cfg.outlier_frac > 0.0:
            raise ValueError("FP4 pools are drawn as bytes; outlier rows do not apply")
        row = (cfg.num_q_heads + 2 * hkv) * d
        qkv_f = _normal_f32(cfg.seed, STAGE_QKV, cfg.num_seqs * row).reshape(cfg.num_seqs, row)
        return Workload(cfg, torch.from_numpy(ctx), torch.from_numpy(bt), draw_fp4_pool(cfg, STAGE_K, nb),
                        draw_fp4_pool(cfg, STAGE_V, nb), _to_storage(qkv_f, cfg.act), None, None)
    pool_shape = (nb, bs, hkv, d)
    kf = _normal_f32(cfg.seed, STAGE_K, int(np.prod(pool_shape))).reshape(pool_shape)
    vf = _normal_f32(cfg.seed, STAGE_V, int(np.prod(pool_shape))).reshape(pool_shape)
    row = (cfg.num_q_heads + 2 * hkv) * d
    qkv_f = _normal_f32(cfg.seed, STAGE_QKV, cfg.num_seqs * row).reshape(cfg.num_seqs, row)

    if cfg.outlier_frac > 0.0:
        # For each (sequence, kv head) exactly floor(frac * ctx) token rows,
        # chosen without replacement, have their K row scaled in fp32.
        kids = _children(cfg.seed, STAGE_OUTLIER, cfg.num_seqs * hkv)
        sc = np.float32(cfg.outlier_scale)
        for b in range(cfg.num_seqs):
            L = int(ctx[b])
            n_out = int(math.floor(cfg.outlier_frac * L))
            for g in range(hkv):
                if n_out == 0:
                    continue
                rng = np.random.default_rng(kids[b * hkv + g])
                toks = rng.choice(L, size=n_out, replace=False)
                pb = bt[b, toks // bs]
                off = toks % bs
                kf[pb, off, g, :] *= sc

    k_scale = v_scale = None
    if cfg.cache == DTYPE_FP8:
        ks, vs = draw_calibration_scales(cfg)
        k_scale, v_scale = torch.from_numpy(ks), torch.from_numpy(vs)
        k_pool = _to_storage(kf, DTYPE_FP8, ks)
        v_pool = _to_storage(vf, DTYPE_FP8, vs)
    else:
        k_pool = _to_storage(kf, cfg.cache)
        v_pool = _to_storage(vf, cfg.cache)
    del kf, vf
    if cfg.cache_layout == "hnd":
        k_pool = k_pool.transpose(1, 2).contiguous()
        v_pool = v_pool.transpose(1, 2).contiguous()
    elif cfg.cache_layout != "nhd":
        raise ValueError(cfg.cache_layout)
    qkv = _to_storage(qkv_f, cfg.act)
    return Workload(cfg, torch.from_numpy(ctx), torch.from_numpy(bt), k_pool, v_pool, qkv, k_scale, v_scale)


def storage_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a host tensor as unsigned integers (uint32/uint16/uint8)."""
    view = {4: torch.int32, 2: torch.int16, 1: torch.uint8}[t.element_size()]
    npy = t.contiguous().view(view).numpy()
    return npy.view({4: np.uint32, 2: np.uint16, 1: np.uint8}[t.element_size()])


def shuffled_copy(w: Workload, seed: int) -> Workload:
    """Same logical cache under a different physical layout: permute the pool's
    blocks and remap the table, so every sequence sees identical rows."""
    nb = w.num_blocks
    perm = torch.from_numpy(np.random.default_rng([seed, 99]).permutation(nb).astype(np.int64))
    # new_pool[perm[i]] = old_pool[i]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    k_new = w.k_pool[inv].clone()
    v_new = w.v_pool[inv].clone()
    bt = w.block_tables.clone()
    mask = bt >= 0
    bt[mask] = perm[bt[mask].long()].to(torch.int32)
    return dataclasses.replace(w, block_tables=bt, k_pool=k_new, v_pool=v_new)


# ------------------------------------------------------------------ multi-head latent attention (MLA)
@dataclasses.dataclass(frozen=True)
class MlaConfig:
    """One paged MLA decode workload: per token a latent of latent_dim values
    (FP8 E4M3 with one static per-tensor scale, or bf16) and a positional part
    of rope_dim bf16 values; num_heads query heads share them.  ``ctx`` is a
    fixed length or an inclusive (lo, hi), as for Config."""

    name: str
    seed: int
    num_seqs: int
    num_heads: int
    ctx: Union[int, Tuple[int, int]]
    partition_size: int
    block_size: int = 64
    latent_dim: int = 512
    rope_dim: int = 64
    ckv_cache: str = DTYPE_FP8
    num_blocks: Optional[int] = None
    calib_tokens: int = 4096
    ctx_list: Optional[Tuple[int, ...]] = None
    description: str = ""

    @property
    def max_ctx(self) -> int:
        if self.ctx_list is not None:
            return max(self.ctx_list) if self.ctx_list else 0
        return self.ctx if isinstance(self.ctx, int) else self.ctx[1]

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_ctx // self.block_size)

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(192): the 128 + 64 query-key width of the models with this cache shape
        return float(np.float32(1.0 / math.sqrt(192.0)))

    def with_(self, **kw) -> "MlaConfig":
        return dataclasses.replace(self, **kw)


MLA_CONFIGS = {
    "mla_kimi_tp8": MlaConfig(
        "mla_kimi_tp8", seed=7, num_seqs=1, num_heads=8, ctx=51200, partition_size=832,
        description="MLA latent decode: 8 heads (one GPU's share of 64 under TP8), 51,200 tokens in 800 pages "
                    "of 64, FP8 E4M3 ckv 512 + bf16 kpe 64, split-K into 62 partitions of 832 tokens"),
    "mla_b16_51k": MlaConfig(
        "mla_b16_51k", seed=8, num_seqs=16, num_heads=8, ctx=51200, partition_size=0,
        description="MLA latent decode at a serving batch: 16 sequences of the same 51,200-token shape, "
                    "library-chosen partitions"),
}


@dataclasses.dataclass
class MlaWorkload:
    cfg: MlaConfig
    context_lens: torch.Tensor  # int32 [B]
    block_tables: torch.Tensor  # int32 [B, MB]
    ckv_pool: torch.Tensor      # [NB, bs, latent_dim] float8_e4m3fn or bfloat16
    kpe_pool: torch.Tensor      # [NB, bs, rope_dim] bfloat16
    q_latent: torch.Tensor      # [B, H, latent_dim] bfloat16
    q_pe: torch.Tensor          # [B, H, rope_dim] bfloat16
    ckv_scale: Optional[torch.Tensor]  # fp32 [1] for an FP8 ckv

    def kv_bytes(self) -> int:
        """Algorithmic bytes one call reads: each token's latent and positional rows once."""
        c = self.cfg
        e = 1 if c.ckv_cache == DTYPE_FP8 else 2
        return int(self.context_lens.clamp(min=0).sum()) * (c.latent_dim * e + c.rope_dim * 2)


def make_mla_workload(cfg: MlaConfig) -> MlaWorkload:
    """Draw order: context lengths, tables, latent rows, positional rows,
    queries, calibration (stage ids as for Config)."""
    ctx = draw_context_lens(cfg)
    bt, nb = draw_block_tables(cfg, ctx)
    bs, dl, dr, B, H = cfg.block_size, cfg.latent_dim, cfg.rope_dim, cfg.num_seqs, cfg.num_heads
    cf = _normal_f32(cfg.seed, STAGE_K, nb * bs * dl).reshape(nb, bs, dl)
    rf = _normal_f32(cfg.seed, STAGE_V, nb * bs * dr).reshape(nb, bs, dr)
    qf = _normal_f32(cfg.seed, STAGE_QKV, B * H * (dl + dr)).reshape(B, H, dl + dr)
    scale = None
    if cfg.ckv_cache == DTYPE_FP8:
        calib = _normal_f32(cfg.seed, STAGE_CALIB, cfg.calib_tokens * dl)
        s = np.float32(np.abs(calib).max()) / np.float32(E4M3_MAX)
        scale = torch.tensor([s], dtype=torch.float32)
        ckv = (torch.from_numpy(cf) / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    elif cfg.ckv_cache == DTYPE_BF16:
        ckv = torch.from_numpy(cf).to(torch.bfloat16)
    else:
        raise ValueError(cfg.ckv_cache)
    kpe = torch.from_numpy(rf).to(torch.bfloat16)
    q = torch.from_numpy(qf).to(torch.bfloat16)
    return MlaWorkload(cfg, torch.from_numpy(ctx), torch.from_numpy(bt), ckv, kpe,
                       q[..., :dl].contiguous(), q[..., dl:].contiguous(), scale)
