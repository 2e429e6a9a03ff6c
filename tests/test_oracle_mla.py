"""Pins for oracle.mla: a library routine (torch SDPA in fp64), split-K
against the unsplit result, closed forms and paging invariants."""
import numpy as np
import torch

import workloads as W
from oracle import attention as A
from oracle import codecs
from oracle import mla as M


def _small(**kw):
    base = dict(num_seqs=3, ctx=(1, 300), partition_size=128, num_blocks=None)
    base.update(kw)
    return W.make_mla_workload(W.MLA_CONFIGS["mla_kimi_tp8"].with_(**base))


def _host(w):
    q_lat = codecs.bf16_decode(W.storage_bits(w.q_latent))
    q_pe = codecs.bf16_decode(W.storage_bits(w.q_pe))
    ckv = W.storage_bits(w.ckv_pool)
    kpe = W.storage_bits(w.kpe_pool)
    s = float(w.ckv_scale[0]) if w.ckv_scale is not None else 1.0
    return q_lat, q_pe, ckv, kpe, s


def _run(w, **kw):
    q_lat, q_pe, ckv, kpe, s = _host(w)
    c = w.cfg
    return M.paged_mla_decode(q_lat, q_pe, ckv, kpe, w.block_tables.numpy(), w.context_lens.numpy(),
                              c.softmax_scale, block_size=c.block_size, ckv_cache=c.ckv_cache, ckv_scale=s, **kw)


def test_matches_torch_sdpa_fp64():
    """MLA is attention whose key is the latent and positional rows side by
    side and whose value is the latent alone: torch's scaled_dot_product
    attention (value width 512, key width 576) in fp64 agrees."""
    w = _small()
    c = w.cfg
    q_lat, q_pe, ckv, kpe, s = _host(w)
    out, lse = _run(w)
    for b in range(c.num_seqs):
        L = int(w.context_lens[b])
        cr, rr = M.gather_latent(ckv, kpe, w.block_tables.numpy(), b, L, c.block_size, c.ckv_cache, s)
        q = torch.from_numpy(np.concatenate([q_lat[b], q_pe[b]], -1))[None]          # [1, H, 576]
        k = torch.from_numpy(np.concatenate([cr, rr], -1))[None, None].expand(1, c.num_heads, L, 576)
        v = torch.from_numpy(cr)[None, None].expand(1, c.num_heads, L, 512)
        ref = torch.nn.functional.scaled_dot_product_attention(q[:, :, None], k, v, scale=c.softmax_scale)
        assert np.abs(out[b] - ref[0, :, 0].numpy()).max() < 1e-12


def test_split_equals_unsplit():
    w = _small(num_seqs=4, ctx=(100, 700))
    c = w.cfg
    q_lat, q_pe, ckv, kpe, s = _host(w)
    out, lse = _run(w)
    for ps in (64, 128, 832):
        o_p, l_p, n = M.paged_mla_partials(q_lat, q_pe, ckv, kpe, w.block_tables.numpy(), w.context_lens.numpy(),
                                          c.softmax_scale, ps, block_size=c.block_size, ckv_cache=c.ckv_cache,
                                          ckv_scale=s)
        mo, ml = A.lse_merge(o_p, l_p, n)
        assert np.abs(mo - out).max() < 1e-12 and np.abs(ml - lse).max() < 1e-12


def test_equal_latent_rows_return_that_row_and_empty_context():
    w = _small(num_seqs=2, ctx_list=(37, 0))
    c = w.cfg
    ckv = w.ckv_pool.view(torch.uint8).clone()
    ckv[:] = torch.from_numpy(np.arange(512) % 120).to(torch.uint8)   # every token's latent is the same row
    w2 = W.MlaWorkload(c, w.context_lens, w.block_tables, ckv.view(torch.float8_e4m3fn), w.kpe_pool, w.q_latent,
                       w.q_pe, w.ckv_scale)
    out, lse = _run(w2)
    row = codecs.e4m3_decode((np.arange(512) % 120).astype(np.uint8)) * np.float64(np.float32(w.ckv_scale[0]))
    assert np.abs(out[0] - row[None]).max() < 1e-12
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()


def test_positional_scores_alone_and_scale_linearity():
    """With q_latent = 0 the scores come from the positional part only, so the
    weights do not depend on ckv_scale and the output scales with it; equal
    positional rows then give the mean latent row."""
    w = _small(num_seqs=2, ctx_list=(50, 129))
    c = w.cfg
    q_lat, q_pe, ckv, kpe, s = _host(w)
    q0 = np.zeros_like(q_lat)
    args = (w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale)
    o1, l1 = M.paged_mla_decode(q0, q_pe, ckv, kpe, *args, block_size=c.block_size, ckv_scale=s)
    o2, l2 = M.paged_mla_decode(q0, q_pe, ckv, kpe, *args, block_size=c.block_size, ckv_scale=2 * s)
    assert np.abs(o2 - 2 * o1).max() < 1e-12 and np.abs(l2 - l1).max() < 1e-12
    kpe_eq = np.broadcast_to(kpe[:1, :1], kpe.shape).copy()
    o3, _ = M.paged_mla_decode(q0, q_pe, ckv, kpe_eq, *args, block_size=c.block_size, ckv_scale=s)
    for b in range(2):
        cr, _ = M.gather_latent(ckv, kpe, args[0], b, int(args[1][b]), c.block_size, "fp8", s)
        assert np.abs(o3[b] - cr.mean(0)[None]).max() < 1e-12


def test_block_shuffle_is_exact():
    w = _small(num_seqs=3, ctx=(10, 400))
    nb = w.ckv_pool.shape[0]
    perm = torch.from_numpy(np.random.default_rng(3).permutation(nb).astype(np.int64))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    bt = w.block_tables.clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    w2 = W.MlaWorkload(w.cfg, w.context_lens, bt, w.ckv_pool[inv].clone(), w.kpe_pool[inv].clone(), w.q_latent,
                       w.q_pe, w.ckv_scale)
    a, b = _run(w), _run(w2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
