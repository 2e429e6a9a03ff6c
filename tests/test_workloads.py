"""The seeded input generator: determinism, shapes and the stated recipes."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def _small(name, **kw):
    return W.CONFIGS[name].with_(**kw)


def test_same_seed_same_bytes_and_different_seed_differs():
    cfg = _small("llama3_8b_gqa", num_seqs=5, ctx=(1, 500))
    a, b = W.make_workload(cfg), W.make_workload(cfg)
    for f in ("context_lens", "block_tables", "k_pool", "v_pool", "qkv"):
        assert torch.equal(getattr(a, f).view(torch.uint8) if getattr(a, f).dtype.is_floating_point else getattr(a, f),
                           getattr(b, f).view(torch.uint8) if getattr(b, f).dtype.is_floating_point else getattr(b, f))
    c = W.make_workload(cfg.with_(seed=99))
    assert not torch.equal(a.qkv.view(torch.int16), c.qkv.view(torch.int16))


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_shapes_dtypes_and_tables(name):
    full = W.CONFIGS[name]
    cfg = full.with_(num_seqs=min(full.num_seqs, 6), ctx=full.ctx if isinstance(full.ctx, int) and full.ctx <= 4096 else
                     ((17, 900) if not isinstance(full.ctx, int) else 1000),
                     num_blocks=full.num_blocks if name != "long_ctx_splitk" else None)
    w = W.make_workload(cfg)
    B, Hq, Hkv, D, bs = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    if cfg.cache == "fp4":
        assert w.k_pool.dtype == torch.uint8 and w.v_pool.dtype == torch.uint8
        assert w.k_pool.shape == (w.num_blocks, W.fp4_block_bytes(bs, Hkv, D)) == w.v_pool.shape
        nc = bs * Hkv * D // 2
        assert set(torch.unique(w.k_pool[:, nc:]).tolist()) <= set(W.FP4_SCALE_BYTES)
        assert w.k_scale is None and w.v_scale is None
    else:
        assert w.k_pool.dtype == W.TORCH_STORAGE[cfg.cache] and w.v_pool.dtype == w.k_pool.dtype
        assert w.k_pool.shape == (w.num_blocks, bs, Hkv, D)
    assert w.qkv.shape == (B, (Hq + 2 * Hkv) * D) and w.qkv.dtype == W.TORCH_STORAGE[cfg.act]
    ctx = w.context_lens.numpy()
    lo, hi = (cfg.ctx, cfg.ctx) if isinstance(cfg.ctx, int) else cfg.ctx
    assert ((ctx >= lo) & (ctx <= hi)).all()
    bt = w.block_tables.numpy()
    seen = []
    for b in range(B):
        n = -(-int(ctx[b]) // bs)
        assert (bt[b, n:] == -1).all()
        assert ((bt[b, :n] >= 0) & (bt[b, :n] < w.num_blocks)).all()
        seen += bt[b, :n].tolist()
    assert len(seen) == len(set(seen)), "physical blocks are distinct across the batch"
    if cfg.cache == "fp8":
        codes = w.k_pool.view(torch.uint8)
        assert not ((codes & 0x7F) == 0x7F).any(), "no NaN codes in the pool"
        assert (w.k_scale > 0).all() and (w.v_scale > 0).all()


def test_tiny_config_uses_an_exact_permutation_of_16_blocks():
    w = W.make_workload(W.CONFIGS["tiny_mqa_f32"])
    assert sorted(w.block_tables[0].tolist()) == list(range(16))
    assert w.block_tables[0].tolist() != list(range(16))


def test_pool_slack_is_a_quarter():
    cfg = _small("llama3_8b_gqa", num_seqs=8, ctx=(100, 1000))
    w = W.make_workload(cfg)
    used = sum(-(-int(c) // 16) for c in w.context_lens)
    assert w.num_blocks == -(-used * 5 // 4)


def test_outlier_rows_are_exactly_one_percent_scaled_by_eight():
    cfg = _small("long_ctx_splitk", num_seqs=2, ctx=3000, num_blocks=None)
    w = W.make_workload(cfg)
    w0 = W.make_workload(cfg.with_(outlier_frac=0.0))
    k = w.k_pool.float()
    k0 = w0.k_pool.float()
    assert torch.equal(w.v_pool.view(torch.int16), w0.v_pool.view(torch.int16))
    for b in range(2):
        for g in range(8):
            rows = []
            for j in range(3000):
                pb, off = int(w.block_tables[b, j // 16]), j % 16
                if not torch.equal(k[pb, off, g], k0[pb, off, g]):
                    assert torch.equal(k[pb, off, g], 8 * k0[pb, off, g])
                    rows.append(j)
            assert len(rows) == math.floor(0.01 * 3000)


def test_calibration_scales_are_absmax_over_448_of_a_gaussian_draw():
    ks, vs = W.draw_calibration_scales(W.CONFIGS["fp8_kv"])
    # absmax of 4096*128 N(0,1) draws lies in [4, 6] with overwhelming probability
    for s in (ks, vs):
        assert s.dtype == np.float32 and s.shape == (8,)
        assert ((s * 448 > 4.0) & (s * 448 < 6.0)).all()
    assert not np.array_equal(ks, vs)


def test_shuffled_copy_keeps_logical_rows():
    cfg = _small("qwen2.5_1.5b_gqa", ctx=100)
    w = W.make_workload(cfg)
    s = W.shuffled_copy(w, 3)
    for b in range(2):
        for j in range(100):
            a = w.k_pool[int(w.block_tables[b, j // 16]), j % 16]
            c = s.k_pool[int(s.block_tables[b, j // 16]), j % 16]
            assert torch.equal(a.view(torch.int16), c.view(torch.int16))
