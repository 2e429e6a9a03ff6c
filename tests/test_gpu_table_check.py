"""lgm_check_block_tables on the GPU: it reports exactly the table entries
and context lengths the decode and append kernels mask or clamp, and the
attention output with such entries is unchanged by the check (the masked
blocks' 16 tokens are left out, as the contract says)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, act_raw, announce, max_abs, out_values, pool_raw, q_from_qkv, to_device
from oracle import attention as OA
from oracle.append import act_to_f64
from paged_gqa_decode_lgm_amd import ops

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _oracle_without_blocks(w, q_raw, bad):
    """Attention over each context with the tokens of the (sequence, logical
    block) pairs in `bad` left out."""
    c = w.cfg
    qf = act_to_f64(np.asarray(q_raw), c.act)
    bt = w.block_tables.numpy().copy()
    for b, lb in bad:
        bt[b, lb] = 0  # a valid id to gather through; its rows are dropped below
    kp = OA.kv_source(pool_raw(w, w.k_pool), c.cache, c.block_size, c.num_kv_heads, c.head_dim)
    vp = OA.kv_source(pool_raw(w, w.v_pool), c.cache, c.block_size, c.num_kv_heads, c.head_dim)
    G = c.num_q_heads // c.num_kv_heads
    out = np.zeros((c.num_seqs, c.num_q_heads, c.head_dim))
    lse = np.zeros((c.num_seqs, c.num_q_heads))
    ctx = w.context_lens.numpy()
    for b in range(c.num_seqs):
        L = int(ctx[b])
        keep = np.ones(L, bool)
        for bb, lb in bad:
            if bb == b:
                keep[lb * c.block_size:(lb + 1) * c.block_size] = False
        for g in range(c.num_kv_heads):
            ks = None if w.k_scale is None else w.k_scale.numpy()
            vs = None if w.v_scale is None else w.v_scale.numpy()
            K = OA.gather_kv(kp, bt, b, L, g, c.block_size, c.cache, ks)[keep]
            V = OA.gather_kv(vp, bt, b, L, g, c.block_size, c.cache, vs)[keep]
            o, ls, _ = OA.attend(qf[b, g * G:(g + 1) * G], K, V, c.softmax_scale)
            out[b, g * G:(g + 1) * G] = o
            lse[b, g * G:(g + 1) * G] = ls
    return out, lse


@pytest.mark.parametrize("name,ps", [("llama3_8b_gqa", 0), ("llama3_8b_gqa", 64), ("fp8_kv", 0)])
def test_check_reports_bad_entries_and_masking_is_unchanged(name, ps):
    cfg = W.CONFIGS[name].with_(num_seqs=6, ctx=(200, 3000), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    mc = d.max_ctx
    st = ops.check_block_tables(d.k_pool, d.block_tables, d.context_lens, mc)
    torch.cuda.synchronize()
    assert st.tolist() == [0, 0, 0, 0]
    # out-of-range entries inside contexts: -1, num_blocks and a huge id
    ctx = w.context_lens.numpy()
    nb = cfg.block_size
    bad = [(1, 3), (1, int(ctx[1] - 1) // nb), (4, 0)]
    vals = [-1, d.k_pool.shape[0], 1 << 30]
    bt = d.block_tables.clone()
    for (b, lb), v in zip(bad, vals):
        bt[b, lb] = v
    announce("table check", name, f"ps={ps}", bad)
    st = ops.check_block_tables(d.k_pool, bt, d.context_lens, mc)
    out, lse = ops.paged_decode_attn(q, d.k_pool, d.v_pool, bt, d.context_lens, mc, softmax_scale=cfg.softmax_scale,
                                     partition_size=ps, k_scale=d.k_scale, v_scale=d.v_scale)
    torch.cuda.synchronize()
    s = st.tolist()
    MB = bt.shape[1]
    assert s[0] == 3 and s[1] == 0
    assert 0x7FFFFFFF - s[2] == 1 * MB + 3  # the first bad (sequence, logical block)
    r_out, r_lse = _oracle_without_blocks(w, act_raw(w, q_from_qkv(w)), bad)
    assert max_abs(out_values(cfg, out), r_out) <= TOL["bf16"]
    g = lse.cpu().numpy().astype(np.float64)
    assert np.abs(g - r_lse).max() <= 1e-4 * max(1.0, np.abs(r_lse).max())
    # a second check adds to the same words
    ops.check_block_tables(d.k_pool, bt, d.context_lens, mc, status=st)
    torch.cuda.synchronize()
    assert st.tolist()[0] == 6


def test_check_reports_clamped_context_lengths():
    cfg = W.CONFIGS["llama3_8b_gqa"].with_(num_seqs=4, ctx=(100, 500), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    ctx = d.context_lens.clone()
    ctx[2] = int(w.context_lens.max()) + 1           # past max_context_len
    ctx[3] = d.block_tables.shape[1] * cfg.block_size + 5  # past the table's capacity
    st = ops.check_block_tables(d.k_pool, d.block_tables, ctx, int(w.context_lens.max()))
    torch.cuda.synchronize()
    assert st.tolist()[1] == 2
