"""A decode step (append of the new token, then attention) captured in a HIP
graph, on every decode plan.  The library only launches kernels on the
caller's stream (no allocation, no memset, no host wait), so a captured
step is the same step: each replay, with eager work and host
synchronisations between the replays, must equal the eager step bitwise
(rotated q, the appended cache bytes, the output and the LSE)."""
import pytest
import torch

import workloads as W
from gpu_util import announce, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

# One case per decode plan the host can choose: whole rows (bf16, FP8, FP4, and the
# single launch of short contexts), whole rows over partitions, work queue, vector ALU.
CASES = {
    "whole_rows_bf16": ("llama3_8b_gqa", dict(num_seqs=8, ctx=(17, 3000))),
    "whole_rows_fp8": ("fp8_kv", dict(num_seqs=8)),
    "whole_rows_fp4": ("fp4_kv", dict(num_seqs=8)),
    "whole_rows_one_launch": ("llama3_8b_gqa", dict(num_seqs=8, ctx=(1, 32))),
    "rows_over_partitions": ("long_ctx_splitk", dict(num_seqs=4, ctx=32768)),
    "work_queue": ("qwen2.5_1.5b_gqa", {}),
    "vector_alu_f32": ("tiny_mqa_f32", {}),
}


def _pool_bytes(pool):
    t = pool.data if hasattr(pool, "data") and not isinstance(pool, torch.Tensor) else pool
    return t.view(torch.uint8).clone()


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_equals_eager_step(case):
    name, over = CASES[case]
    base = W.CONFIGS[name]
    if over and base.num_blocks is None:
        over = {**over, "num_blocks": None}
    cfg = base.with_(**over)
    w = W.make_workload(cfg)
    d = to_device(w)
    B, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    mc = d.max_ctx
    from paged_gqa_decode_lgm_amd import ops

    q = torch.empty((B, Hq, D), dtype=d.qkv.dtype, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws_bytes = ops.workspace_bytes(q, d.k_pool, d.block_tables, mc, cfg.partition_size)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        ops.rope_kv_append(d.qkv, d.k_pool, d.v_pool, d.block_tables, d.context_lens, cfg.rope_theta, Hq,
                           d.k_scale, d.v_scale, q_out=q)
        ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                              softmax_scale=cfg.softmax_scale, partition_size=cfg.partition_size,
                              k_scale=d.k_scale, v_scale=d.v_scale, out=out, out_lse=lse, workspace=ws)

    announce("graph", case, cfg.name)
    step()  # the append rewrites the same slots with the same bytes: the step is idempotent
    torch.cuda.synchronize()
    ref = (q.clone(), out.clone(), lse.clone(), _pool_bytes(d.k_pool), _pool_bytes(d.v_pool))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    other = torch.empty_like(out)
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        q.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        got = (q, out, lse, _pool_bytes(d.k_pool), _pool_bytes(d.v_pool))
        for g, r, what in zip(got, ref, ("q", "out", "lse", "k_pool", "v_pool")):
            assert torch.equal(g.view(torch.uint8), r.view(torch.uint8)), f"replay {i}: {what} differs"
        # eager work of the program between the replays: an attention call into other buffers
        ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                              softmax_scale=cfg.softmax_scale, partition_size=cfg.partition_size,
                              k_scale=d.k_scale, v_scale=d.v_scale, out=other)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.uint8), ref[1].view(torch.uint8))
