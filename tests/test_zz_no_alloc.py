"""The allocation-free attention entry point (lgm_paged_decode_attn_static,
include/lgm.h) against lgm_paged_decode_attn through the C ABI: on every
plan, two calls in a row (the second with a smaller input, so the shared
device array holds the first call's contents when the second starts) give
bitwise the outputs and LSEs of the workspace entry point on the same
inputs, and those match the oracle within the bar."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, act_raw, announce, max_abs, oracle_attention, out_values, pool_raw, q_from_qkv, to_device
from paged_gqa_decode_lgm_amd import ops

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

# (workload, first input, second (smaller) input, partition size)
CASES = [
    ("llama3_8b_gqa", dict(num_seqs=16, ctx=(4500, 5000)), dict(num_seqs=5, ctx=(1, 900)), 0),     # ranges, then single launch
    ("llama3_8b_gqa", dict(num_seqs=16, ctx=(17, 5000)), dict(num_seqs=5, ctx=(1, 900)), 64),      # work queue
    ("qwen2.5_1.5b_gqa", dict(), dict(num_seqs=1, ctx_list=(700,)), 64),                          # work queue, Hkv 2
    ("qwen2.5_1.5b_gqa", dict(), dict(num_seqs=1, ctx_list=(700,)), 0),                           # single launch
    ("qwen2.5_1.5b_gqa", dict(num_seqs=320), dict(num_seqs=3, ctx_list=(40, 300, 2048)), 0),       # token slices
    ("fp8_kv", dict(num_seqs=24), dict(num_seqs=3, ctx=(40, 300)), 0),
    ("fp4_kv", dict(num_seqs=24), dict(num_seqs=3, ctx=(40, 300)), 0),
    ("long_ctx_splitk", dict(num_seqs=2, ctx=40000), dict(num_seqs=1, ctx=20000), 512),          # row partitions
    ("tiny_mqa_f32", dict(), dict(ctx_list=(100,)), 0),                                           # vector ALU
    ("tiny_mqa_f32", dict(num_seqs=3, ctx_list=(256, 1000, 3)), dict(ctx_list=(40,)), 64),         # split, merge
]


def _inputs(name, over):
    over = dict(over)
    if over:
        over.setdefault("num_blocks", None)  # a pool sized for the new contexts
    cfg = W.CONFIGS[name].with_(append=False, **over)
    w = W.make_workload(cfg)
    return w, to_device(w), q_from_qkv(w).cuda()


def _call_both(w, d, q, ps):
    c = w.cfg
    mc = d.max_ctx
    kw = dict(softmax_scale=c.softmax_scale, partition_size=ps, k_scale=d.k_scale, v_scale=d.v_scale)
    o_s, l_s = ops.paged_decode_attn_static(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc, **kw)
    o_w, l_w = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc, **kw)
    torch.cuda.synchronize()
    return o_s, l_s, o_w, l_w


@pytest.mark.parametrize("name,first,second,ps", CASES)
def test_static_entry_matches_workspace_entry(name, first, second, ps):
    for which, over in (("first", first), ("second", second)):
        w, d, q = _inputs(name, over)
        announce("static entry", name, which, f"B={w.cfg.num_seqs}", f"max_ctx={d.max_ctx}", f"ps={ps}")
        o_s, l_s, o_w, l_w = _call_both(w, d, q, ps)
        assert torch.equal(o_s.view(torch.uint8), o_w.view(torch.uint8)), (name, which, "outputs differ")
        assert torch.equal(l_s.view(torch.int32), l_w.view(torch.int32)), (name, which, "LSEs differ")
        r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
        assert max_abs(out_values(w.cfg, o_s), r_out) <= TOL[w.cfg.act]
        g = l_s.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(g), np.isneginf(r_lse))
        fin = np.isfinite(r_lse)
        assert np.abs(g[fin] - r_lse[fin]).max() <= 1e-4 * max(1.0, np.abs(r_lse[fin]).max())


def test_static_entry_repeats_bitwise():
    """Back-to-back calls on one stream (no host sync between them) leave the
    work counters zero for the next: four work-queue calls give one result."""
    w, d, q = _inputs("llama3_8b_gqa", dict(num_seqs=12, ctx=(1, 3000)))
    c = w.cfg
    outs = [ops.paged_decode_attn_static(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                         softmax_scale=c.softmax_scale, partition_size=64) for _ in range(4)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16)) and torch.equal(l, outs[0][1])
