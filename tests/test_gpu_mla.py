"""GPU parity of the paged MLA decode (include/lgm_mla.h) against the fp64
oracle (oracle.mla) on the same seeded inputs.

Bar: max-abs <= 2e-2 on the bf16 outputs (as for the other bf16 / FP8
attention paths), LSE within 1e-4 relative, -inf exactly where the oracle
has it; index handling (poisoned unused slots and table entries, repeated
calls) bitwise identical.  The mainarch README's MLA gates check every
eight-wide window of the 512-element latent output and a ragged page and
split boundary: the full-size test reports the error per window, and the
edge tests put partition ends inside pages and contexts one token past or
short of a page.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce
from oracle import codecs
from oracle import mla as OM
from paged_gqa_decode_lgm_amd import ops

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

TOL = 2e-2
BASE = W.MLA_CONFIGS["mla_kimi_tp8"]
EDGE_CTX = (0, 1, 31, 63, 64, 65, 200, 833, 1000, 2100)


def _dev(w):
    cu = lambda t: None if t is None else t.to("cuda")
    return dict(q_latent=cu(w.q_latent), q_pe=cu(w.q_pe), ckv=cu(w.ckv_pool), kpe=cu(w.kpe_pool),
                bt=cu(w.block_tables), ctx=cu(w.context_lens), scale=cu(w.ckv_scale))


def _gpu(w, d, ps, max_ctx=None, **kw):
    mc = int(w.context_lens.max()) if max_ctx is None else max_ctx
    return ops.paged_mla_decode(d["q_latent"], d["q_pe"], d["ckv"], d["kpe"], d["bt"], d["ctx"], mc,
                                w.cfg.softmax_scale, d["scale"], partition_size=ps, **kw)


def _oracle(w, seqs=None, ckv_bits=None, kpe_bits=None):
    c = w.cfg
    q_lat = codecs.bf16_decode(W.storage_bits(w.q_latent))
    q_pe = codecs.bf16_decode(W.storage_bits(w.q_pe))
    ckv = W.storage_bits(w.ckv_pool) if ckv_bits is None else ckv_bits
    kpe = W.storage_bits(w.kpe_pool) if kpe_bits is None else kpe_bits
    return OM.paged_mla_decode(q_lat, q_pe, ckv, kpe, w.block_tables.numpy(), w.context_lens.numpy(),
                               c.softmax_scale, block_size=c.block_size, ckv_cache=c.ckv_cache,
                               ckv_scale=float(w.ckv_scale[0]), seqs=seqs)


def _check(w, out, lse, seqs=None):
    r_out, r_lse = _oracle(w, seqs)
    rows = list(range(w.cfg.num_seqs)) if seqs is None else list(seqs)
    g = out.float().cpu().numpy()[rows]
    r = r_out[rows]
    err = np.abs(g - r).max() if g.size else 0.0
    announce(w.cfg.name, f"B={w.cfg.num_seqs} H={w.cfg.num_heads} bs={w.cfg.block_size}", "max-abs", err)
    assert err <= TOL, err
    gl = lse.cpu().numpy().astype(np.float64)[rows]
    rl = r_lse[rows]
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    if fin.any():
        assert np.abs(gl[fin] - rl[fin]).max() <= 1e-4 * max(1.0, np.abs(rl[fin]).max())
    return g, r


@pytest.mark.parametrize("ps", [0, 32, 96, 832, 4096])
@pytest.mark.parametrize("bs", [64, 16, 1])
def test_ragged_page_and_split_edges(ps, bs):
    """Contexts around page ends (block_size +-1) and partitions that end
    inside pages (96 with pages of 64, 832 = 13 pages, 32 inside pages of 64)."""
    cfg = BASE.with_(name=f"mla_edge_bs{bs}_ps{ps}", seed=21, num_seqs=len(EDGE_CTX), ctx_list=EDGE_CTX,
                     block_size=bs, partition_size=ps)
    w = W.make_mla_workload(cfg)
    d = _dev(w)
    out, lse = _gpu(w, d, ps)
    torch.cuda.synchronize()
    g, _ = _check(w, out, lse)
    assert np.all(g[0] == 0.0)  # the empty context writes zeros


@pytest.mark.parametrize("H", [1, 5, 8, 16])
def test_head_counts(H):
    cfg = BASE.with_(name=f"mla_heads{H}", seed=22, num_seqs=4, ctx=(1, 3000), num_heads=H)
    w = W.make_mla_workload(cfg)
    d = _dev(w)
    out, lse = _gpu(w, d, 0)
    torch.cuda.synchronize()
    _check(w, out, lse)


@pytest.mark.parametrize("ps", [0, 832])
def test_full_size_every_latent_window(ps):
    """The full workload (51,200 tokens in 800 pages, 8 heads) in the
    benchmark's launch configuration (library-chosen partitions) and with
    the 832-token partitions; every eight-wide window of every head's
    512-element output within the bar."""
    w = W.make_mla_workload(BASE)
    d = _dev(w)
    out, lse = _gpu(w, d, ps)
    torch.cuda.synchronize()
    g, r = _check(w, out, lse)
    win = np.abs(g - r).reshape(g.shape[0], g.shape[1], 64, 8).max(axis=(0, 1, 3))
    announce("mla full size", f"ps={ps}", "worst window", int(win.argmax()), float(win.max()))
    assert win.shape == (64,) and np.all(win <= TOL)


def test_full_size_batch_every_sequence():
    """The 16-sequence serving workload in the benchmark's launch
    configuration; the oracle checks every sequence."""
    w = W.make_mla_workload(W.MLA_CONFIGS["mla_b16_51k"])
    d = _dev(w)
    out, lse = _gpu(w, d, 0)
    torch.cuda.synchronize()
    _check(w, out, lse)


def test_poisoned_unused_slots_and_entries_are_bitwise_identical():
    """Slots past each context (NaN codes 0x7F, bf16 NaN in kpe), unused
    pool blocks and table entries past each context (out-of-range ids) do
    not change a bit of the result."""
    cfg = BASE.with_(name="mla_poison", seed=23, num_seqs=len(EDGE_CTX), ctx_list=EDGE_CTX, partition_size=96)
    w = W.make_mla_workload(cfg)
    d = _dev(w)
    out0, lse0 = _gpu(w, d, 96)
    ckv = d["ckv"].view(torch.uint8).clone()
    kpe = d["kpe"].view(torch.int16).clone()
    bt = w.block_tables.clone()
    bs = cfg.block_size
    used = set()
    for b, L in enumerate(EDGE_CTX):
        nb = -(-L // bs)
        used |= set(bt[b, :nb].tolist())
        if L % bs:
            last = int(bt[b, nb - 1])
            ckv[last, L % bs:] = 0x7F
            kpe[last, L % bs:] = 0x7FC0
        bt[b, nb:] = 10 ** 6
    for blk in range(ckv.shape[0]):
        if blk not in used:
            ckv[blk] = 0x7F
            kpe[blk] = 0x7FC0
    d2 = dict(d, ckv=ckv.view(torch.float8_e4m3fn), kpe=kpe.view(torch.bfloat16), bt=bt.cuda())
    out1, lse1 = _gpu(w, d2, 96)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))


def test_repeated_calls_and_workspace_reuse_are_bitwise_identical():
    cfg = BASE.with_(name="mla_repeat", seed=24, num_seqs=3, ctx=(500, 5000))
    w = W.make_mla_workload(cfg)
    d = _dev(w)
    mc = int(w.context_lens.max())
    need = ops.mla_workspace_bytes(d["q_latent"], d["q_pe"], d["ckv"], d["bt"], mc, 0)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # no zeroing needed
    out0, lse0 = _gpu(w, d, 0, workspace=ws)
    out1, lse1 = _gpu(w, d, 0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))
    _check(w, out0, lse0)


def test_lse_optional_and_max_context_len_clamp():
    """out_lse may be NULL; contexts above max_context_len are clamped to it."""
    cfg = BASE.with_(name="mla_clamp", seed=25, num_seqs=3, ctx_list=(300, 700, 1200))
    w = W.make_mla_workload(cfg)
    d = _dev(w)
    out, lse = _gpu(w, d, 0, want_lse=False)
    assert lse is None
    torch.cuda.synchronize()
    ref, _ = _gpu(w, d, 0)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    out_c, lse_c = _gpu(w, d, 0, max_ctx=700)
    torch.cuda.synchronize()
    wc = dataclasses.replace(w, context_lens=torch.tensor([300, 700, 700], dtype=torch.int32))
    _check(wc, out_c, lse_c)
