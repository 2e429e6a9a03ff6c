"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.

Tolerances (the bar):
  attention outputs   max-abs <= 1e-5 (fp32 activations), <= 2e-2 (bf16 / FP8 paths)
  appended entries    within 1 bf16 ulp of the exact rotation (ord distance),
                      fp32 caches within the fp32 rounding bound of the rotation
  FP8 cache bytes     bit-exact against the oracle's fp32 recipe
  index handling      bit-exact: every other pool byte unchanged, block-shuffle
                      and poisoned-slot runs bitwise identical
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (TOL, act_raw, act_raw_tensor, announce, bf16_ord, gpu_append, gpu_attention, host_bits,
                      max_abs, oracle_append, oracle_attention, out_values, pool_raw, q_from_qkv, to_device)
from oracle import attention as OA
from oracle import codecs
from paged_gqa_decode_lgm_amd import ops

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

# Sizes the oracle finishes in seconds that still span several partitions and a ragged tail.
PARITY = {
    "tiny_mqa_f32": {},
    "qwen2.5_1.5b_gqa": {},
    "llama3_8b_gqa": dict(num_seqs=8, ctx=(17, 2000)),
    "long_ctx_splitk": dict(num_seqs=2, ctx=8192),
    "fp8_kv": dict(num_seqs=8),
    "fp4_kv": dict(num_seqs=8),
}


def _host_pool(pool):
    """A device pool back on the host (FP4 pools are wrapped)."""
    return (pool.data if isinstance(pool, ops.FP4Pool) else pool).cpu()


def _lse_check(g_lse, r_lse, rows=None):
    g = np.asarray(g_lse, np.float64)
    r = np.asarray(r_lse, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert np.array_equal(np.isneginf(g), np.isneginf(r))
    fin = np.isfinite(r)
    if fin.any():
        assert np.abs(g[fin] - r[fin]).max() <= 1e-4 * max(1.0, np.abs(r[fin]).max())


def _pair_abs(x):
    """|x_i| + |x_{i+D/2}| for every element of rows x [.., D] (both halves)."""
    h = x.shape[-1] // 2
    a = np.abs(x[..., :h]) + np.abs(x[..., h:])
    return np.concatenate([a, a], -1)


def _pair_abs_interleaved(x):
    """|x_2i| + |x_2i+1| for both elements of every adjacent pair."""
    a = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    return np.repeat(a, 2, axis=-1)


def _check_bf16_rotation(g_bits, rec_bits, exact, pair_abs):
    """Rotated bf16 values: within 1 ord of the fp32-recipe mirror, and within
    one bf16 ulp plus the fp32 recipe's rounding bound (4 * 2^-24 * (|x_i| +
    |x_i+D/2|), |cos|, |sin| <= 1) of the exact rotation.  Under cancellation
    (x_i cos ~ x_i+D/2 sin) that bound exceeds one bf16 ulp of the tiny
    result, and no fp32 evaluation can do better."""
    assert np.abs(bf16_ord(g_bits) - bf16_ord(rec_bits)).max() <= 1
    g = codecs.bf16_decode(np.asarray(g_bits, np.uint16)).astype(np.float64)
    _, e = np.frexp(g)
    ulp = np.where(g == 0, 2.0 ** -133, np.ldexp(1.0, e - 8))
    assert (np.abs(g - exact) <= ulp + 4 * 2.0 ** -24 * pair_abs).all()


def _check_append(w, d, q_gpu, rec, ex, seqs=None):
    """q_out and the appended cache slots against the oracle; all other pool bytes unchanged."""
    c = w.cfg
    seqs = range(c.num_seqs) if seqs is None else seqs
    gq = act_raw_tensor(c, q_gpu)
    gk = pool_raw(w, _host_pool(d.k_pool))
    gv = pool_raw(w, _host_pool(d.v_pool))
    k0, v0 = pool_raw(w, w.k_pool), pool_raw(w, w.v_pool)
    slots = {s for s in rec.slots if s is not None}
    if c.cache != "fp4" and c.cache_layout == "hnd":
        # compare through [NB, bs, Hkv, D] views of the head-major pools
        sw = lambda a: np.swapaxes(a, 1, 2)
        gk, gv, k0, v0 = sw(gk), sw(gv), sw(k0), sw(v0)
        rec = dataclasses.replace(rec, k_pool=sw(rec.k_pool), v_pool=sw(rec.v_pool))
        ex = dataclasses.replace(ex, k_pool=sw(ex.k_pool), v_pool=sw(ex.v_pool))
    if c.cache == "fp4":
        # every byte of both pools: the MX codes and scale bytes of the recipe
        # at the target slots, everything else unchanged
        assert np.array_equal(gk, rec.k_pool), "FP4 K pool bytes"
        assert np.array_equal(gv, rec.v_pool), "FP4 V pool bytes"
    else:
        # index exactness: only the target slots moved
        mask = np.ones(gk.shape[:2], bool)
        for (pb, off) in slots:
            mask[pb, off] = False
        assert np.array_equal(gk[mask], k0[mask]) and np.array_equal(gv[mask], v0[mask])
    xq = xk = None
    if c.act == "bf16":
        x = codecs.bf16_decode(W.storage_bits(w.qkv)).astype(np.float64)
        Hq, Hkv, D = c.num_q_heads, c.num_kv_heads, c.head_dim
        xq = x[:, : Hq * D].reshape(-1, Hq, D)
        xk = x[:, Hq * D:(Hq + Hkv) * D].reshape(-1, Hkv, D)
    pair_abs = _pair_abs if c.rope_style == "neox" else _pair_abs_interleaved
    for b in seqs:
        if c.act == "bf16":
            _check_bf16_rotation(gq[b], rec.q_out[b], ex.q_rot[b], pair_abs(xq[b]))
        else:
            x = w.qkv.numpy()[b, : c.num_q_heads * c.head_dim].astype(np.float64).reshape(c.num_q_heads, -1)
            bound = 4 * 2.0 ** -24 * pair_abs(x)
            assert (np.abs(gq[b].astype(np.float64) - ex.q_rot[b]) <= bound).all()
        if rec.slots[b] is None or c.cache == "fp4":
            continue
        pb, off = rec.slots[b]
        if c.cache == "fp8":
            assert np.array_equal(gk[pb, off], rec.k_pool[pb, off]), f"K bytes, seq {b}"
            assert np.array_equal(gv[pb, off], rec.v_pool[pb, off]), f"V bytes, seq {b}"
        elif c.cache == "bf16":
            _check_bf16_rotation(gk[pb, off], rec.k_pool[pb, off], ex.k_rot[b], pair_abs(xk[b]))
            assert np.abs(bf16_ord(gv[pb, off]) - bf16_ord(ex.v_pool[pb, off])).max() <= 1
        else:
            assert np.abs(gk[pb, off] - ex.k_pool[pb, off]).max() <= 4 * 2.0 ** -24 * 8
            assert np.array_equal(gv[pb, off], ex.v_pool[pb, off])


def _run_and_check(cfg, sample=None, partition_size=None):
    w = W.make_workload(cfg)
    announce(cfg.name, f"B={cfg.num_seqs}", f"Hq/Hkv={cfg.num_q_heads}/{cfg.num_kv_heads}", f"D={cfg.head_dim}",
             f"cache={cfg.cache}", f"max_ctx={int(w.context_lens.max())}", f"ps={cfg.partition_size}")
    d = to_device(w)
    if cfg.append:
        q = gpu_append(d)
    else:
        q = q_from_qkv(w).cuda()
    out, lse = gpu_attention(d, q, partition_size)
    torch.cuda.synchronize()
    if cfg.append:
        rec = oracle_append(w, "recipe")
        ex = oracle_append(w, "exact")
        _check_append(w, d, q, rec, ex, sample)
        q_ref, kp, vp = rec.q_out, rec.k_pool, rec.v_pool
    else:
        q_ref, kp, vp = act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool)
    r_out, r_lse = oracle_attention(w, q_ref, kp, vp, seqs=sample)
    rows = slice(None) if sample is None else list(sample)
    err = max_abs(out_values(cfg, out), r_out, rows)
    announce(cfg.name, "max-abs", err)
    assert err <= TOL[cfg.act], err
    _lse_check(lse.cpu().numpy(), r_lse, rows)
    return w, d, out, lse


@pytest.mark.parametrize("name", list(PARITY))
def test_config_parity(name):
    base = W.CONFIGS[name]
    over = dict(PARITY[name])
    if over and base.num_blocks is None:
        over["num_blocks"] = None
    _run_and_check(base.with_(**over))


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "long_ctx_splitk", "fp8_kv", "fp4_kv"])
def test_full_size_every_sequence(name):
    """Full-size workload in the launch configuration the benchmark times
    (the append, then attention with the workload's partition size): every
    output element of every sequence against the oracle, so every split
    point of the equal tile ranges and every partition boundary is covered."""
    _run_and_check(W.CONFIGS[name])


EDGE_CTX = (0, 1, 15, 16, 17, 63, 64, 65, 200, 513)


@pytest.mark.parametrize("act,cache,D,G", [
    ("bf16", "bf16", 128, 4), ("bf16", "bf16", 128, 6), ("bf16", "bf16", 128, 1), ("bf16", "bf16", 64, 8),
    ("bf16", "fp8", 128, 4), ("bf16", "fp8", 64, 3), ("f32", "f32", 64, 4), ("f32", "f32", 128, 2),
    ("bf16", "bf16", 128, 8), ("bf16", "fp8", 128, 5), ("bf16", "fp4", 128, 4), ("bf16", "fp4", 128, 7),
])
@pytest.mark.parametrize("ps", [16, 64, 0, 4096])
def test_shapes_and_ragged_edges(act, cache, D, G, ps):
    cfg = W.Config(f"edge_{act}_{cache}_D{D}_G{G}", seed=11, num_seqs=len(EDGE_CTX), num_q_heads=2 * G,
                   num_kv_heads=2, head_dim=D, block_size=16, act=act, cache=cache, ctx=0, rope_theta=1e4,
                   partition_size=ps, append=True, ctx_list=EDGE_CTX)
    _run_and_check(cfg)


def _bench_like(name="llama3_8b_gqa", **kw):
    base = W.CONFIGS[name]
    return base.with_(**{"num_blocks": None, **kw})


def test_block_shuffle_is_bitwise_identical():
    cfg = _bench_like(num_seqs=6, ctx=(100, 3000), append=False)
    w = W.make_workload(cfg)
    w2 = W.shuffled_copy(w, 7)
    q = q_from_qkv(w).cuda()
    announce("shuffle", cfg.name)
    o1, l1 = gpu_attention(to_device(w), q)
    o2, l2 = gpu_attention(to_device(w2), q)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_poisoned_unused_slots_and_table_entries_are_bitwise_identical():
    cfg = _bench_like(num_seqs=6, ctx=(100, 3000), append=False)
    w = W.make_workload(cfg)
    q = q_from_qkv(w).cuda()
    bt = w.block_tables.clone()
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    used = set()
    for b in range(cfg.num_seqs):
        L = int(w.context_lens[b])
        nb = -(-L // 16)
        used |= set(bt[b, :nb].tolist())
        bt[b, nb:] = torch.tensor([-5, 1 << 30] * bt.shape[1], dtype=torch.int32)[: bt.shape[1] - nb]
        last = int(bt[b, nb - 1])
        kp[last, L - (nb - 1) * 16:] = float("nan")
        vp[last, L - (nb - 1) * 16:] = float("nan")
    unused = [i for i in range(kp.shape[0]) if i not in used]
    kp[unused] = float("nan")
    vp[unused] = float("inf")
    w2 = dataclasses.replace(w, block_tables=bt, k_pool=kp, v_pool=vp)
    announce("poison", cfg.name)
    o1, l1 = gpu_attention(to_device(w), q)
    o2, l2 = gpu_attention(to_device(w2), q)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_repeated_calls_are_bitwise_identical():
    cfg = _bench_like(num_seqs=16, ctx=(512, 8192), append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    announce("determinism x20", cfg.name)
    o0, l0 = gpu_attention(d, q)
    for _ in range(19):
        o, l = gpu_attention(d, q)
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)) and torch.equal(l, l0)


def test_out_lse_optional_and_strided_q():
    cfg = _bench_like(num_seqs=3, ctx=(40, 700), append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    qd = q_from_qkv(w).cuda()
    padded = torch.zeros((3, 33, 128), dtype=qd.dtype, device="cuda")
    padded[:, :32] = qd
    qs = padded[:, :32]  # sequence stride 33*128
    announce("strided q / no lse", cfg.name)
    o1, _ = ops.paged_decode_attn(qs, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                  softmax_scale=cfg.softmax_scale, want_lse=False)
    o2, _ = gpu_attention(d, qd)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_fp8_every_code_decodes_exactly():
    """V rows hold every finite E4M3 code; equal keys make the output the mean of
    the decoded V rows, which the oracle computes from the codes' definition."""
    cfg = W.CONFIGS["fp8_kv"].with_(num_seqs=2, ctx_list=(254, 254), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vb = w.v_pool.view(torch.uint8).clone()
    kb = torch.full_like(w.k_pool.view(torch.uint8), 0x38)
    for b in range(2):
        for j in range(254):
            pb = int(w.block_tables[b, j // 16])
            vb[pb, j % 16] = torch.from_numpy(np.roll(codes, j + 3 * b)[:128].copy())
    w2 = dataclasses.replace(w, k_pool=kb.view(torch.float8_e4m3fn), v_pool=vb.view(torch.float8_e4m3fn))
    q = q_from_qkv(w2).cuda()
    announce("fp8 all codes")
    out, lse = gpu_attention(to_device(w2), q)
    torch.cuda.synchronize()
    r_out, r_lse = oracle_attention(w2, act_raw(w2, q_from_qkv(w2)), pool_raw(w2, w2.k_pool), pool_raw(w2, w2.v_pool))
    assert max_abs(out_values(cfg, out), r_out) <= TOL["bf16"]
    _lse_check(lse.cpu().numpy(), r_lse)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_standalone(out_dtype):
    rng = np.random.default_rng(5)
    B, H, P, D = 5, 6, 37, 128
    po = rng.standard_normal((B, H, P, D)).astype(np.float32)
    pl = (rng.standard_normal((B, H, P)) * 6).astype(np.float32)
    pl[1, :, 3] = -np.inf
    pl[2] = -np.inf                     # a sequence whose records are all empty
    # empty records weigh exactly zero whatever their rows hold
    po[1, :, 3] = np.nan
    po[2, :, ::2] = np.inf
    po[2, :, 1::2] = np.nan
    pl[4, :, 0] = -np.inf               # n = 1 and that record empty
    po[4, :, 0, :7] = -np.inf
    n = np.array([37, 5, 37, 0, 1], np.int32)
    announce("lse_merge", out_dtype)
    out, lse = ops.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                             torch.from_numpy(n).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    r_out, r_lse = OA.lse_merge(po, pl, n)
    g = out.float().cpu().numpy().astype(np.float64)
    tol = 1e-5 if out_dtype == torch.float32 else 2e-2
    assert np.isfinite(g).all() and np.isfinite(r_out).all()
    assert np.abs(g - r_out).max() <= tol
    _lse_check(lse.cpu().numpy(), r_lse)
    # without counts: every record is used
    out2, _ = ops.lse_merge(torch.from_numpy(po[:2]).cuda(), torch.from_numpy(pl[:2]).cuda(), None, out_dtype=out_dtype)
    r2, _ = OA.lse_merge(po[:2], pl[:2])
    assert np.abs(out2.float().cpu().numpy() - r2).max() <= tol


def test_inactive_sequence_append_writes_nothing():
    cfg = W.CONFIGS["qwen2.5_1.5b_gqa"].with_(num_seqs=3, ctx_list=(0, 5, 2048))
    w = W.make_workload(cfg)
    d = to_device(w)
    announce("inactive append")
    q = gpu_append(d)
    torch.cuda.synchronize()
    rec = oracle_append(w, "recipe")
    ex = oracle_append(w, "exact")
    _check_append(w, d, q, rec, ex)
    assert np.array_equal(act_raw_tensor(cfg, q)[0], W.storage_bits(w.qkv)[0, : 12 * 128].reshape(12, 128))


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "fp8_kv", "fp4_kv"])
@pytest.mark.parametrize("ps", [64, 128])
def test_persistent_workspace_is_reusable_and_left_zeroed(name, ps):
    """The matrix-core kernel hands out work items from two counters at the
    start of the workspace: a zero-filled workspace reused by consecutive calls
    must give identical results and be left with both counters back at zero."""
    cfg = W.CONFIGS[name].with_(num_seqs=12, ctx=(1, 3000), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    mc = d.max_ctx
    nbytes = ops.workspace_bytes(q, d.k_pool, d.block_tables, mc, ps)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    announce("persistent workspace reuse", name, ps, nbytes)
    outs = []
    for _ in range(3):
        o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                                     softmax_scale=cfg.softmax_scale, partition_size=ps, k_scale=d.k_scale,
                                     v_scale=d.v_scale, workspace=ws)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16)) and torch.equal(l, outs[0][1])
    assert int(ws[:4096].view(torch.int32).abs().sum()) == 0
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
    assert max_abs(out_values(cfg, outs[0][0]), r_out) <= TOL["bf16"]
    _lse_check(outs[0][1].cpu().numpy(), r_lse)


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "fp8_kv"])
def test_one_workspace_serves_every_plan(name):
    """One zero-filled workspace shared by calls on different plans in turn:
    equal ranges (partition_size 0), the whole-row partition plan, the work
    queue (partitions of 64) and equal ranges again.  Of these plans only
    the work queue touches the counter slot at its start, and it leaves the
    slot zero, so every call matches the oracle and the slot ends at zero
    (the single-launch plan, which also counts there, is covered with the
    work queue below)."""
    cfg = W.CONFIGS[name].with_(num_seqs=12, ctx=(1, 20000), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    mc = d.max_ctx
    plans = [0, 256, 64, 0, 64]
    assert ops.partition_size(q, d.k_pool, d.block_tables, mc, 0) == 0  # equal ranges
    nbytes = max(ops.workspace_bytes(q, d.k_pool, d.block_tables, mc, ps) for ps in plans)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    announce("shared workspace across plans", name, plans, nbytes)
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
    for ps in plans:
        o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                                     softmax_scale=cfg.softmax_scale, partition_size=ps, k_scale=d.k_scale,
                                     v_scale=d.v_scale, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4096].view(torch.int32).abs().sum()) == 0, ps
        assert max_abs(out_values(cfg, o), r_out) <= TOL["bf16"], ps
        _lse_check(l.cpu().numpy(), r_lse)


@pytest.mark.parametrize("ps", [0, 16, 32])
def test_many_short_sequences_and_empty_ones(ps):
    """Short and zero-length contexts across more than three 64-sequence chunks
    of the work-item walk, with one to several items per sequence; and a
    batch with fewer work items than workgroups."""
    ctx = tuple([0, 1, 5, 31, 32, 33, 0, 64, 100, 17] * 21)
    cfg = W.CONFIGS["llama3_8b_gqa"].with_(num_seqs=len(ctx), ctx_list=ctx, num_blocks=None, append=False,
                                           partition_size=ps)
    _run_and_check(cfg)
    cfg1 = W.CONFIGS["qwen2.5_1.5b_gqa"].with_(num_seqs=1, ctx_list=(40,), num_blocks=None, append=False)
    _run_and_check(cfg1)


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("hkv,G", [(4, 1), (4, 4), (8, 4), (8, 5), (16, 2), (8, 11), (8, 12), (8, 16)])
def test_row_plan_ragged_edges(cache, hkv, G):
    """Whole-row ranges (partition_size 0, kv heads divisible by 4): head
    groups of 4 and 8, empty and one-token contexts, block and tile edges.
    FP4 at 11 and 12 query heads per kv head: the two sides of the bound on
    its eight-wave workgroup shape.
    The edge contexts twice over and one 16384-token context: past the
    single-launch plan's tile cap (16384 tiles, 32768 for FP8)."""
    ctx = EDGE_CTX * 2 + (16384,)
    cfg = W.Config(f"rows_{cache}_H{hkv}_G{G}", seed=12, num_seqs=len(ctx), num_q_heads=hkv * G,
                   num_kv_heads=hkv, head_dim=128, block_size=16, act="bf16", cache=cache, ctx=0, rope_theta=1e4,
                   partition_size=0, append=True, ctx_list=ctx)
    assert len(ctx) * hkv * 16384 // 32 > 32768
    _run_and_check(cfg)


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("hkv,G", [(2, 6), (1, 8), (6, 4), (1, 16), (2, 1), (3, 5)])
def test_row_plan_token_slices(cache, hkv, G):
    """Whole-row ranges over head groups of 2 and 1 kv heads (num_kv_heads
    not divisible by 4): each head's steps are dealt to 2 or 4 waves in
    interleaved token slices whose partial results the flush combines.
    Contexts shorter than the slices (slices that see no token), step counts
    that are no multiple of the slice count, and a long context split across
    ranges; enough sequences to pass the single-launch caps."""
    ctx = EDGE_CTX * 7 + (16384,)
    cfg = W.Config(f"slices_{cache}_H{hkv}_G{G}", seed=18, num_seqs=len(ctx), num_q_heads=hkv * G,
                   num_kv_heads=hkv, head_dim=128, block_size=16, act="bf16", cache=cache, ctx=0, rope_theta=1e4,
                   partition_size=0, append=True, ctx_list=ctx)
    assert len(ctx) * hkv * 16384 // 32 > 32768
    _run_and_check(cfg)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("hkv,G,B", [(2, 6, 320), (1, 8, 640)])
def test_row_plan_token_slices_full_size(cache, hkv, G, B):
    """Token slices past the single-launch caps at the shapes timed for them
    (Qwen2.5-1.5B-shaped 12/2 and an MQA 8/1, 2048-token contexts; 256 and
    512 sequences reach the FP8 cap exactly, so a few more): every output
    element of every sequence against the oracle."""
    cfg = W.CONFIGS["qwen2.5_1.5b_gqa"].with_(name=f"slices_full_{cache}_H{hkv}_G{G}", num_seqs=B, num_kv_heads=hkv,
                                              num_q_heads=hkv * G, cache=cache, num_blocks=None)
    assert B * hkv * 2048 // 32 > 32768  # past the single-launch caps (16384 tiles, 32768 for FP8)
    _run_and_check(cfg)


# ------------------------------------------------------------------ single-launch plan
# partition_size 0 with at most 1022 (sequence, kv head) streams and at most 16384
# 32-token tiles over them (32768 for FP8): one launch, partitions of whole
# 128-token steps, the last workgroup to finish one of a context's partitions
# merges its records.
def _single_launch_cfg(name, cache, hkv, G, ctx, seed=16, append=True):
    cfg = W.Config(name, seed=seed, num_seqs=len(ctx), num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=128,
                   block_size=16, act="bf16", cache=cache, ctx=0, rope_theta=1e4, partition_size=0, append=append,
                   ctx_list=tuple(ctx))
    streams, tiles = len(ctx) * hkv, len(ctx) * hkv * -(-max(ctx) // 32)
    assert streams <= 1022 and tiles <= 16384, (streams, tiles)
    return cfg


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("hkv,G", [(1, 16), (2, 6), (4, 1), (1, 8), (3, 5)])
def test_single_launch_ragged_edges(cache, hkv, G):
    """Empty, one-token, block-edge and step-edge contexts next to ones of
    several partitions: contexts written directly (one partition) and merged
    ones (up to 5 partitions) in one grid."""
    ctx = EDGE_CTX + (128, 129, 640, 383)
    _run_and_check(_single_launch_cfg(f"single_{cache}_H{hkv}_G{G}", cache, hkv, G, ctx))


@pytest.mark.parametrize("hkv,ctx", [(1, 65536), (2, 32768), (1, 65535), (2, 20001)])
def test_single_launch_many_partitions_and_steps(hkv, ctx):
    """Up to 64 partitions per context (the most the plan makes), of 4 to 8
    steps per wave: the merge reads its records in several batches."""
    cfg = _single_launch_cfg(f"single_long_H{hkv}_{ctx}", "bf16", hkv, 8, (ctx,), seed=17, append=False)
    _run_and_check(cfg)


def test_single_launch_counters_left_zero_and_workspace_shared():
    """The arrival counters (the counter slot's words 2..) come back zero
    after every call, so calls repeat bitwise, and the work-queue plan may
    use the same workspace in between."""
    cfg = W.CONFIGS["qwen2.5_1.5b_gqa"].with_(num_seqs=3, ctx_list=(2048, 700, 1), num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    nbytes = max(ops.workspace_bytes(q, d.k_pool, d.block_tables, d.max_ctx, ps) for ps in (0, 64))
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    announce("single-launch counters", nbytes)
    outs = []
    for ps in (0, 0, 64, 0, 64, 0):
        o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                     softmax_scale=cfg.softmax_scale, partition_size=ps, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4096].view(torch.int32).abs().sum()) == 0, ps
        outs.append((ps, o.clone(), l.clone()))
    ref = [x for x in outs if x[0] == 0][0]
    for ps, o, l in outs:
        if ps == 0:
            assert torch.equal(o.view(torch.int16), ref[1].view(torch.int16)) and torch.equal(l, ref[2])
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
    for ps, o, l in outs:
        assert max_abs(out_values(cfg, o), r_out) <= TOL["bf16"], ps
        _lse_check(l.cpu().numpy(), r_lse)


def test_single_launch_back_to_back_different_inputs():
    """Calls with different queries, caches and context lengths on one
    workspace, no host sync between them: each call's merges see its own
    records and arrival counts."""
    cfgs = [W.CONFIGS["qwen2.5_1.5b_gqa"].with_(seed=50 + i, num_seqs=2, ctx_list=c, num_blocks=None, append=False)
            for i, c in enumerate([(2048, 2048), (1000, 2047), (129, 1920)])]
    ws_list = [W.make_workload(c) for c in cfgs]
    devs = [to_device(w) for w in ws_list]
    qs = [q_from_qkv(w).cuda() for w in ws_list]
    nbytes = max(ops.workspace_bytes(q, d.k_pool, d.block_tables, d.max_ctx, 0) for q, d in zip(qs, devs))
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    announce("single-launch back-to-back", nbytes)
    outs = []
    for rep in range(3):
        for q, d, c in zip(qs, devs, cfgs):
            outs.append(ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                              softmax_scale=c.softmax_scale, partition_size=0, workspace=ws))
    torch.cuda.synchronize()
    assert int(ws[:4096].view(torch.int32).abs().sum()) == 0
    for i, (w, c) in enumerate(zip(ws_list, cfgs)):
        r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
        for rep in range(3):
            o, l = outs[rep * len(cfgs) + i]
            assert max_abs(out_values(c, o), r_out) <= TOL["bf16"]
            _lse_check(l.cpu().numpy(), r_lse)


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp4"])
def test_row_plan_short_contexts_single_launch(cache):
    """Every context within one 32-token tile (max_context_len 32): no stream
    can be split, so the call is the decode launch alone, and the decode
    kernel itself writes the empty contexts (out = 0, lse = -inf).  130
    sequences x 8 kv heads: past the single-launch plan's 1022 streams."""
    ctx = (0, 1, 5, 16, 17, 31, 32, 0, 2, 32) * 13
    cfg = W.Config(f"rows_short_{cache}", seed=15, num_seqs=len(ctx), num_q_heads=32, num_kv_heads=8, head_dim=128,
                   block_size=16, act="bf16", cache=cache, ctx=0, rope_theta=5e5, partition_size=0, append=True,
                   ctx_list=ctx)
    w, d, out, lse = _run_and_check(cfg)
    assert torch.count_nonzero(out[0]).item() == 0 and torch.count_nonzero(out[7]).item() == 0
    assert bool(torch.isneginf(lse[0]).all()) and bool(torch.isneginf(lse[7]).all())


def test_row_plan_more_workgroups_than_tiles():
    """The range count follows the longest context, so one long sequence among
    many one-token ones leaves most ranges empty, between non-empty ones."""
    ctx = (8192,) + (1,) * 40 + (0, 33, 17) + (1,) * 20
    cfg = _bench_like(num_seqs=len(ctx), ctx_list=ctx, append=False, partition_size=0)
    _run_and_check(cfg)


def test_row_plan_many_sequences_scan_chunks():
    """More sequences than one scan step of the range walk (1024)."""
    ctx = tuple((i * 37) % 97 for i in range(1100))
    cfg = W.Config("rows_many", seed=13, num_seqs=len(ctx), num_q_heads=8, num_kv_heads=4, head_dim=128,
                   block_size=16, act="bf16", cache="bf16", ctx=0, rope_theta=1e4, partition_size=0, append=False,
                   ctx_list=ctx)
    _run_and_check(cfg)


def test_row_plan_workspace_reuse():
    """The row plan needs no zeroed workspace (every entry it reads is written
    earlier in the same call): a reused, non-zero one gives identical results."""
    ctx = (1, 3000, 6000, 17, 500, 2048, 4095, 33, 5000, 1, 600, 3333)  # 96 streams x 188 tiles: whole-row plan
    cfg = W.CONFIGS["llama3_8b_gqa"].with_(num_seqs=len(ctx), ctx_list=ctx, num_blocks=None, append=False)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    assert ops.partition_size(q, d.k_pool, d.block_tables, d.max_ctx, 0) == 0
    nbytes = ops.workspace_bytes(q, d.k_pool, d.block_tables, d.max_ctx, 0)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    ws[:4096] = 0  # the counter slot: zero on entry for every plan
    announce("row workspace reuse", nbytes)
    outs = []
    for _ in range(3):
        o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                     softmax_scale=cfg.softmax_scale, partition_size=0, workspace=ws)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16)) and torch.equal(l, outs[0][1])
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
    assert max_abs(out_values(cfg, outs[0][0]), r_out) <= TOL["bf16"]
    _lse_check(outs[0][1].cpu().numpy(), r_lse)


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "long_ctx_splitk"])
def test_row_plan_back_to_back_different_inputs(name):
    """Calls with different queries and caches on one workspace, no host sync
    between them: each must see its own split records, not the previous
    call's."""
    # past the single-launch plan's tile cap: the whole-row ranges
    over = dict(num_seqs=10, ctx=(7000, 16000)) if name == "llama3_8b_gqa" else dict(num_seqs=2, ctx=40000)
    cfgs = [W.CONFIGS[name].with_(seed=40 + i, num_blocks=None, append=False, partition_size=0, **over)
            for i in range(3)]
    ws_list = [W.make_workload(c) for c in cfgs]
    devs = [to_device(w) for w in ws_list]
    qs = [q_from_qkv(w).cuda() for w in ws_list]
    mc = max(d.max_ctx for d in devs)
    nbytes = max(ops.workspace_bytes(q, d.k_pool, d.block_tables, mc, 0) for q, d in zip(qs, devs))
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    announce("row plan back-to-back", name, nbytes)
    outs = []
    for rep in range(2):
        for q, d, c in zip(qs, devs, cfgs):
            o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, mc,
                                         softmax_scale=c.softmax_scale, partition_size=0, workspace=ws)
            outs.append((o, l))
    torch.cuda.synchronize()
    for i, (w, c) in enumerate(zip(ws_list, cfgs)):
        r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
        for rep in range(2):
            o, l = outs[rep * len(cfgs) + i]
            assert max_abs(out_values(c, o), r_out) <= TOL["bf16"]
            _lse_check(l.cpu().numpy(), r_lse)


@pytest.mark.gpu
def test_stream_read_probe_reads_without_writing():
    """The streaming-ceiling probe only reads: its sink is left alone for a
    buffer whose words XOR to zero, and the buffer is unchanged."""
    from paged_gqa_decode_lgm_amd import _binding as Bn
    nbytes = 8 * 16384 * 4
    announce("stream read probe", nbytes)
    buf = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    for nt in (0, 1):
        Bn.lgm_stream_read_probe(buf, nbytes, 8, nt, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == -5
    assert bool((buf == 7).all())


# ------------------------------------------------------------------ FP4 caches
def _fp4_parts(pool: torch.Tensor, cfg):
    """Code and scale views of an FP4 pool tensor [NB, block_bytes] (host or device)."""
    bs, hkv, d = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    nc = bs * hkv * d // 2
    return pool[:, :nc].view(-1, bs, hkv, d // 2), pool[:, nc:].view(-1, bs, hkv, d // 32)


@pytest.mark.parametrize("ps", [0, 64])
def test_fp4_poisoned_unused_slots_and_blocks_are_bitwise_identical(ps):
    """Slots past each context and blocks no table uses hold code bytes 0xFF
    and NaN scale bytes (0xFF); table entries past the context are out of
    range.  None of it may reach the output."""
    cfg = W.CONFIGS["fp4_kv"].with_(num_seqs=6, ctx=(100, 3000), num_blocks=None, append=False,
                                    partition_size=ps)
    w = W.make_workload(cfg)
    q = q_from_qkv(w).cuda()
    bt = w.block_tables.clone()
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    used = set()
    for pool in (kp, vp):
        codes, scales = _fp4_parts(pool, cfg)
        for b in range(cfg.num_seqs):
            L = int(w.context_lens[b])
            nb = -(-L // 16)
            used |= set(w.block_tables[b, :nb].tolist())
            last = int(w.block_tables[b, nb - 1])
            codes[last, L - (nb - 1) * 16:] = 0xFF
            scales[last, L - (nb - 1) * 16:] = 0xFF
    for b in range(cfg.num_seqs):
        nb = -(-int(w.context_lens[b]) // 16)
        bt[b, nb:] = torch.tensor([-5, 1 << 30] * bt.shape[1], dtype=torch.int32)[: bt.shape[1] - nb]
    unused = [i for i in range(kp.shape[0]) if i not in used]
    kp[unused] = 0xFF
    vp[unused] = 0xFF
    w2 = dataclasses.replace(w, block_tables=bt, k_pool=kp, v_pool=vp)
    announce("fp4 poison", ps)
    o1, l1 = gpu_attention(to_device(w), q, ps)
    o2, l2 = gpu_attention(to_device(w2), q, ps)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool))
    assert max_abs(out_values(cfg, o1), r_out) <= TOL["bf16"]


@pytest.mark.parametrize("ps", [0, 64])
def test_fp4_every_code_and_scale_position_decodes_exactly(ps):
    """K rows all decode to 1.0 (code 0x2, scale byte 127), so every key is
    equal and the output is the mean of the V rows.  V rows cycle through all
    16 codes in every nibble position with scale bytes 0x00 (2^-127) and
    120..127 in every scale position; the oracle decodes them from the
    format's definition."""
    cfg = W.CONFIGS["fp4_kv"].with_(num_seqs=2, ctx_list=(254, 254), num_blocks=None, append=False,
                                    partition_size=ps)
    w = W.make_workload(cfg)
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    kc, ks = _fp4_parts(kp, cfg)
    kc[:] = 0x22
    ks[:] = 127
    vc, vs = _fp4_parts(vp, cfg)
    rng = np.random.default_rng(17)
    for b in range(2):
        for j in range(254):
            pb, off = int(w.block_tables[b, j // 16]), j % 16
            lo = (np.arange(64) + j + 5 * b) % 16
            hi = (np.arange(64) * 7 + 3 * j + b) % 16
            vc[pb, off] = torch.from_numpy((lo | (hi << 4)).astype(np.uint8)).view(1, 64).expand(cfg.num_kv_heads, 64)
            vs[pb, off] = torch.from_numpy(rng.choice([0, 120, 121, 122, 123, 124, 125, 126, 127],
                                                      size=(cfg.num_kv_heads, 4)).astype(np.uint8))
    w2 = dataclasses.replace(w, k_pool=kp, v_pool=vp)
    q = q_from_qkv(w2).cuda()
    announce("fp4 all codes", ps)
    out, lse = gpu_attention(to_device(w2), q, ps)
    torch.cuda.synchronize()
    r_out, r_lse = oracle_attention(w2, act_raw(w2, q_from_qkv(w2)), pool_raw(w2, w2.k_pool), pool_raw(w2, w2.v_pool))
    assert max_abs(out_values(cfg, out), r_out) <= TOL["bf16"]
    _lse_check(lse.cpu().numpy(), r_lse)


def test_fp4_append_quantises_edge_blocks_exactly():
    """New K/V rows whose 32-element blocks hit the rounding edges: exact
    midpoints between codes, values above 6 * scale, an all-zero block and a
    block of negative values that round to zero; the bytes must equal the
    oracle's."""
    cfg = W.CONFIGS["fp4_kv"].with_(num_seqs=4, ctx_list=(1, 17, 300, 16), num_blocks=None)
    w = W.make_workload(cfg)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    qkv = w.qkv.float().numpy().reshape(cfg.num_seqs, Hq + 2 * Hkv, D)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -0.75, -5.0, -7.5, 6.0, 4.0, 0.5, 0.0])
    for b in range(cfg.num_seqs):
        for g in range(Hkv):
            v = qkv[b, Hq + Hkv + g]
            v[0:16] = mids * 2.0 ** (g - 3)         # block 0: midpoints at scale 2^(g-3) (largest 7.5 -> X = g - 3)
            v[16:32] = mids[::-1] * 2.0 ** (g - 3)
            v[32:64] = 0.0                          # block 1: all zero
            v[64:96] = -(2.0 ** -12)                # block 2: tiny negatives (round to -0 against a big value)
            v[96] = 3.0
    qb = torch.from_numpy(qkv.reshape(cfg.num_seqs, -1)).to(torch.bfloat16)
    w2 = dataclasses.replace(w, qkv=qb)
    d = to_device(w2)
    announce("fp4 append edges")
    q = gpu_append(d)
    torch.cuda.synchronize()
    rec = oracle_append(w2, "recipe")
    ex = oracle_append(w2, "exact")
    _check_append(w2, d, q, rec, ex)


@pytest.mark.parametrize("D", [8, 24, 40, 96])
@pytest.mark.parametrize("act,cache", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "fp8")])
def test_append_small_and_odd_head_dims(D, act, cache):
    """Head dims whose half is not a multiple of 8 take the element-wise path
    even with aligned buffers; every rotated value and appended slot must
    still match the oracle (the append supports any even D up to 256)."""
    cfg = W.Config(f"append_D{D}_{cache}", seed=21, num_seqs=5, num_q_heads=6, num_kv_heads=2, head_dim=D,
                   block_size=16, act=act, cache=cache, ctx=0, rope_theta=1e4, partition_size=0, append=True,
                   ctx_list=(1, 16, 17, 40, 0))
    w = W.make_workload(cfg)
    d = to_device(w)
    announce("append", cfg.name)
    q = gpu_append(d)
    torch.cuda.synchronize()
    _check_append(w, d, q, oracle_append(w, "recipe"), oracle_append(w, "exact"))


# ------------------------------------------------------------------ contract variants
VARIANTS = [
    # (cache, layout, rope_style, per_tensor, partition_size, hkv, G)
    ("bf16", "hnd", "neox", False, 0, 8, 4),          # whole-row plan, head-major blocks
    ("bf16", "hnd", "interleaved", False, 64, 2, 6),  # work-queue plan
    ("bf16", "nhd", "interleaved", False, 0, 4, 4),
    ("fp8", "hnd", "neox", True, 0, 8, 4),
    ("fp8", "nhd", "interleaved", True, 64, 2, 5),
    ("fp8", "hnd", "interleaved", False, 32, 4, 1),   # MHA sibling (G = 1)
    ("fp4", "hnd", "neox", False, 0, 8, 4),           # eight-wave FP4 row plan
    ("fp4", "hnd", "interleaved", False, 64, 2, 4),
    ("f32", "hnd", "interleaved", False, 64, 1, 4),   # vector-ALU plan, D = 64
]


@pytest.mark.parametrize("cache,layout,rope_style,per_tensor,ps,hkv,G", VARIANTS)
def test_contract_variants(cache, layout, rope_style, per_tensor, ps, hkv, G):
    """Interleaved RoPE, head-major (HND) blocks and per-tensor FP8 scales,
    append then attention, over the plans and cache dtypes, ragged contexts."""
    D = 64 if cache == "f32" else 128
    cfg = W.Config(f"variant_{cache}_{layout}_{rope_style}_{'pt' if per_tensor else 'ph'}", seed=31,
                   num_seqs=len(EDGE_CTX), num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, block_size=16,
                   act="f32" if cache == "f32" else "bf16", cache=cache, ctx=0, rope_theta=1e4, partition_size=ps,
                   append=True, ctx_list=EDGE_CTX, rope_style=rope_style, cache_layout=layout,
                   scale_per_tensor=per_tensor)
    _run_and_check(cfg)


# ------------------------------------------------------------------ whole-row partition plan
@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("hkv,G,ps", [(8, 4, 256), (4, 4, 256), (16, 2, 512), (8, 16, 256), (2, 6, 256), (6, 2, 512)])
def test_row_partition_plan_ragged_edges(cache, hkv, G, ps):
    """Explicit partition sizes of whole tiles (>= 256 tokens) on whole-row
    shapes with a long context (>= 64 partitions) in the batch: equal runs of
    whole partitions, a record per partition of a split context, merged by
    lse_merge; empty, one-token and tile-edge contexts and contexts that are a
    partition plus one token."""
    ctx = EDGE_CTX + (ps + 1, 2 * ps, 3 * ps - 17, 64 * ps + 5) + (ps // 2,) * 20
    cfg = W.Config(f"rowparts_{cache}_H{hkv}_G{G}_ps{ps}", seed=14, num_seqs=len(ctx), num_q_heads=hkv * G,
                   num_kv_heads=hkv, head_dim=128, block_size=16, act="bf16", cache=cache, ctx=0, rope_theta=1e4,
                   partition_size=ps, append=True, ctx_list=ctx)
    _run_and_check(cfg)


def test_row_partition_plan_needs_no_zeroed_workspace_and_many_sequences():
    """The partition plan reads only records written earlier in the same call
    (a 0x7F-filled workspace gives identical results on repeated calls), and
    walks more sequences than one scan step (1024)."""
    ctx = tuple((i * 131) % 1500 for i in range(1099)) + (16400,)   # one context of 65 partitions
    cfg = W.Config("rowparts_many", seed=15, num_seqs=len(ctx), num_q_heads=8, num_kv_heads=4, head_dim=128,
                   block_size=16, act="bf16", cache="bf16", ctx=0, rope_theta=1e4, partition_size=256, append=False,
                   ctx_list=ctx)
    w = W.make_workload(cfg)
    d = to_device(w)
    q = q_from_qkv(w).cuda()
    assert ops.partition_size(q, d.k_pool, d.block_tables, d.max_ctx, 256) == 256
    nbytes = ops.workspace_bytes(q, d.k_pool, d.block_tables, d.max_ctx, 256)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    announce("row partition plan, 1100 sequences", nbytes)
    outs = []
    for _ in range(2):
        o, l = ops.paged_decode_attn(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_ctx,
                                     softmax_scale=cfg.softmax_scale, partition_size=256, workspace=ws)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16)) and torch.equal(outs[0][1], outs[1][1])
    sample = list(range(0, 1100, 37)) + [1099]
    r_out, r_lse = oracle_attention(w, act_raw(w, q_from_qkv(w)), pool_raw(w, w.k_pool), pool_raw(w, w.v_pool),
                                    seqs=sample)
    assert max_abs(out_values(cfg, outs[0][0]), r_out, sample) <= TOL["bf16"]
    _lse_check(outs[0][1].cpu().numpy(), r_lse, sample)
