"""Pins for oracle.append: slot arithmetic, rounding bounds against the exact
rotation, FP8 bytes against the codec, inactive sequences."""
import numpy as np
import pytest
import torch

import workloads
from oracle import append as AP
from oracle import codecs, rope


def _wl(name, **kw):
    return workloads.make_workload(workloads.CONFIGS[name].with_(**kw))


def _append(w, mode):
    c = w.cfg
    raw = (lambda t: t.numpy()) if c.cache == "f32" else workloads.storage_bits
    qkv = w.qkv.numpy() if c.act == "f32" else workloads.storage_bits(w.qkv)
    return AP.rope_kv_append(
        qkv, w.context_lens.numpy(), w.block_tables.numpy(), raw(w.k_pool), raw(w.v_pool),
        num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
        block_size=c.block_size, act=c.act, cache=c.cache, rope_theta=c.rope_theta,
        k_scale=None if w.k_scale is None else w.k_scale.numpy(),
        v_scale=None if w.v_scale is None else w.v_scale.numpy(), mode=mode)


def bf16_ord(bits):
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


@pytest.mark.parametrize("name", ["tiny_mqa_f32", "qwen2.5_1.5b_gqa", "fp8_kv"])
def test_only_target_slots_change(name):
    w = _wl(name, num_seqs=min(4, workloads.CONFIGS[name].num_seqs), num_blocks=None)
    r = _append(w, "recipe")
    c = w.cfg
    raw = (lambda t: t.numpy()) if c.cache == "f32" else workloads.storage_bits
    k0, v0 = raw(w.k_pool), raw(w.v_pool)
    changed_k = np.argwhere((r.k_pool != k0).any(axis=(2, 3)))
    expect = set()
    for b in range(c.num_seqs):
        pos = int(w.context_lens[b]) - 1
        pb = int(w.block_tables[b, pos // c.block_size])
        assert r.slots[b] == (pb, pos % c.block_size)
        expect.add((pb, pos % c.block_size))
    assert {tuple(x) for x in changed_k.tolist()} <= expect
    changed_v = np.argwhere((r.v_pool != v0).any(axis=(2, 3)))
    assert {tuple(x) for x in changed_v.tolist()} <= expect


def test_bf16_recipe_within_one_ulp_of_exact():
    w = _wl("qwen2.5_1.5b_gqa")
    r = _append(w, "recipe")
    e = _append(w, "exact")
    assert np.abs(bf16_ord(r.q_out) - bf16_ord(e.q_out)).max() <= 1
    for (pb, off) in r.slots:
        assert np.abs(bf16_ord(r.k_pool[pb, off]) - bf16_ord(e.k_pool[pb, off])).max() <= 1
        assert np.array_equal(r.v_pool[pb, off], e.v_pool[pb, off])  # bf16 -> bf16 is a copy


def test_bf16_v_is_copied_and_k_is_the_rotation():
    w = _wl("qwen2.5_1.5b_gqa")
    c = w.cfg
    r = _append(w, "exact")
    x = codecs.bf16_decode(workloads.storage_bits(w.qkv)).reshape(c.num_seqs, c.num_q_heads + 2 * c.num_kv_heads, c.head_dim)
    for b in range(c.num_seqs):
        pb, off = r.slots[b]
        assert np.array_equal(codecs.bf16_decode(r.v_pool[pb, off]), x[b, c.num_q_heads + c.num_kv_heads:])
        k = rope.rope_neox_f64(x[b, c.num_q_heads:c.num_q_heads + c.num_kv_heads], 2047, c.rope_theta)
        assert np.array_equal(r.k_pool[pb, off], codecs.bf16_encode(k))


def test_f32_recipe_error_bound_against_exact():
    """fp32 recipe vs the exact rotation: two rounded products and a rounded
    sum, with cos/sin each within half an ulp, give an error below
    4 * 2^-24 * (|x_i| + |x_{i+D/2}|) (relative to the terms, since the sum
    can cancel)."""
    w = _wl("tiny_mqa_f32")
    r = _append(w, "recipe")
    e = _append(w, "exact")
    c = w.cfg
    x = w.qkv.numpy().astype(np.float64).reshape(1, -1, c.head_dim)
    h = c.head_dim // 2
    mag = lambda v: np.concatenate([np.abs(v[..., :h]) + np.abs(v[..., h:])] * 2, axis=-1)
    bound_q = 4 * 2.0 ** -24 * mag(x[:, :4])
    assert (np.abs(r.q_out.astype(np.float64) - e.q_rot) <= bound_q).all()
    pb, off = r.slots[0]
    assert pb == int(w.block_tables[0, 255 // 16]) and off == 15
    bound_k = 4 * 2.0 ** -24 * mag(x[0, 4:5])
    assert (np.abs(r.k_pool[pb, off].astype(np.float64) - e.k_rot[0]) <= bound_k).all()
    assert np.array_equal(r.v_pool[pb, off], w.qkv.numpy()[0, 5 * 64:6 * 64].reshape(1, 64))


def test_fp8_bytes_are_the_codec_of_the_recipe():
    w = _wl("fp8_kv", num_seqs=16, num_blocks=None)
    c = w.cfg
    r = _append(w, "recipe")
    ks, vs = w.k_scale.numpy(), w.v_scale.numpy()
    x = codecs.bf16_decode(workloads.storage_bits(w.qkv)).reshape(c.num_seqs, -1, c.head_dim)
    n_zero = 0
    for b in range(c.num_seqs):
        pb, off = r.slots[b]
        pos = int(w.context_lens[b]) - 1
        k32 = rope.rope_neox_f32_recipe(x[b, 32:40].astype(np.float32), pos, c.rope_theta)
        kq = np.divide(k32, ks[:, None], dtype=np.float32)
        assert np.array_equal(r.k_pool[pb, off], codecs.e4m3_encode(kq))
        vq = np.divide(x[b, 40:48].astype(np.float32), vs[:, None], dtype=np.float32)
        assert np.array_equal(r.v_pool[pb, off], codecs.e4m3_encode(vq))
        # quantisation error bound: half the local code spacing (or saturation)
        dec = codecs.e4m3_decode(r.k_pool[pb, off])
        a = np.minimum(np.abs(kq.astype(np.float64)), 448.0)
        spacing = np.where(a < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2 ** -6))) - 3))
        assert (np.abs(np.abs(dec) - a) <= spacing / 2 + 1e-12).all()
        n_zero += int((r.k_pool[pb, off] & 0x7F == 0).sum())


def test_inactive_sequence_writes_nothing_and_copies_q():
    w = _wl("qwen2.5_1.5b_gqa")
    w.context_lens[0] = 0
    r = _append(w, "recipe")
    assert r.slots[0] is None
    qbits = workloads.storage_bits(w.qkv)[0, : 12 * 128].reshape(12, 128)
    assert np.array_equal(r.q_out[0], qbits)
    pb, off = r.slots[1]
    k0 = workloads.storage_bits(w.k_pool)
    changed = np.argwhere((r.k_pool != k0).any(axis=(2, 3)))
    assert [tuple(x) for x in changed.tolist()] == [(pb, off)]


def test_fp4_append_writes_mx_codes_of_the_recipe_and_nothing_else():
    """Each active sequence's new K row (fp32 recipe rotation) and V row are
    written as MX FP4: codes at (slot * Hkv + g) * D/2 of the block, scale
    bytes at bs * Hkv * D/2 + (slot * Hkv + g) * D/32; every other byte of
    both pools is unchanged."""
    w = _wl("fp4_kv", num_seqs=12, ctx=(1, 200), num_blocks=None)
    c = w.cfg
    w.context_lens[3] = 0
    r = _append(w, "recipe")
    hkv, d, bs = c.num_kv_heads, c.head_dim, c.block_size
    nc = bs * hkv * d // 2
    x = codecs.bf16_decode(workloads.storage_bits(w.qkv)).reshape(c.num_seqs, -1, d)
    k_expect = workloads.storage_bits(w.k_pool).copy()
    v_expect = workloads.storage_bits(w.v_pool).copy()
    for b in range(c.num_seqs):
        if r.slots[b] is None:
            assert int(w.context_lens[b]) <= 0
            continue
        pb, off = r.slots[b]
        pos = int(w.context_lens[b]) - 1
        assert (pb, off) == (int(w.block_tables[b, pos // bs]), pos % bs)
        k32 = rope.rope_neox_f32_recipe(x[b, 32:40].astype(np.float32), pos, c.rope_theta)
        for expect, rows in ((k_expect, k32.astype(np.float64)), (v_expect, x[b, 40:48])):
            codes, sc = codecs.mx_fp4_quantize(rows)
            packed = codecs.fp4_pack(codes)
            for g in range(hkv):
                expect[pb, (off * hkv + g) * d // 2:(off * hkv + g + 1) * d // 2] = packed[g]
                expect[pb, nc + (off * hkv + g) * d // 32:nc + (off * hkv + g + 1) * d // 32] = sc[g]
    assert np.array_equal(r.k_pool, k_expect)
    assert np.array_equal(r.v_pool, v_expect)


# ------------------------------------------------------------------ contract variants
def _append_raw(w, mode, **kw):
    c = w.cfg
    raw = (lambda t: t.numpy()) if c.cache == "f32" else workloads.storage_bits
    qkv = w.qkv.numpy() if c.act == "f32" else workloads.storage_bits(w.qkv)
    return AP.rope_kv_append(
        qkv, w.context_lens.numpy(), w.block_tables.numpy(), kw.pop("k_pool", raw(w.k_pool)),
        kw.pop("v_pool", raw(w.v_pool)), num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
        head_dim=c.head_dim, block_size=c.block_size, act=c.act, cache=c.cache, rope_theta=c.rope_theta,
        k_scale=kw.pop("k_scale", None if w.k_scale is None else w.k_scale.numpy()),
        v_scale=kw.pop("v_scale", None if w.v_scale is None else w.v_scale.numpy()), mode=mode, **kw)


@pytest.mark.parametrize("mode", ["recipe", "exact"])
def test_interleaved_append_is_neox_append_of_even_odd_split_rows(mode):
    """Permuting each Q and K head's elements (evens first, then odds) and
    running the NeoX append gives, after undoing the permutation, exactly the
    interleaved append: q_out and the appended K rows bit for bit, V as is."""
    w = _wl("qwen2.5_1.5b_gqa", num_seqs=3, ctx=(1, 300), num_blocks=None)
    c = w.cfg
    D, Hq, Hkv = c.head_dim, c.num_q_heads, c.num_kv_heads
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    qkv = workloads.storage_bits(w.qkv).reshape(c.num_seqs, Hq + 2 * Hkv, D).copy()
    qkv_p = qkv.copy()
    qkv_p[:, :Hq + Hkv] = qkv[:, :Hq + Hkv][..., perm]
    w_p = workloads.Workload(c, w.context_lens, w.block_tables, w.k_pool, w.v_pool,
                             torch.from_numpy(qkv_p.reshape(c.num_seqs, -1)).view(torch.bfloat16), None, None)
    r_int = _append_raw(w, mode, rope_style="interleaved")
    r_neo = _append_raw(w_p, mode)
    assert np.array_equal(r_int.q_out, r_neo.q_out[..., inv])
    for b in range(c.num_seqs):
        pb, off = r_int.slots[b]
        assert np.array_equal(r_int.k_pool[pb, off], r_neo.k_pool[pb, off][..., inv])
        assert np.array_equal(r_int.v_pool[pb, off], r_neo.v_pool[pb, off])


@pytest.mark.parametrize("name", ["qwen2.5_1.5b_gqa", "fp8_kv", "fp4_kv", "tiny_mqa_f32"])
def test_hnd_append_writes_the_same_rows_head_major(name):
    """Appending into HND pools equals appending into NHD pools and then
    moving every block's rows head-major (the conversion is written out in
    test_oracle_attention)."""
    import test_oracle_attention as T_A
    over = dict(num_seqs=6, ctx=(1, 200), num_blocks=None) if name != "tiny_mqa_f32" else {}
    w = _wl(name, **over)
    c = w.cfg
    raw = (lambda t: t.numpy()) if c.cache == "f32" else workloads.storage_bits
    if c.cache == "fp4":
        conv = lambda p: T_A._fp4_to_hnd(p, c.block_size, c.num_kv_heads, c.head_dim)
    else:
        conv = T_A._to_hnd
    r_nhd = _append_raw(w, "recipe")
    r_hnd = _append_raw(w, "recipe", k_pool=conv(raw(w.k_pool)), v_pool=conv(raw(w.v_pool)), layout="hnd")
    assert np.array_equal(r_hnd.q_out, r_nhd.q_out)
    assert np.array_equal(r_hnd.k_pool, conv(r_nhd.k_pool)) and np.array_equal(r_hnd.v_pool, conv(r_nhd.v_pool))


def test_per_tensor_fp8_append_uses_the_one_scale_for_every_head():
    w = _wl("fp8_kv", num_seqs=8, num_blocks=None)
    one = _append_raw(w, "recipe", k_scale=np.array([0.0123], np.float32), v_scale=np.array([0.0234], np.float32))
    each = _append_raw(w, "recipe", k_scale=np.full(8, 0.0123, np.float32), v_scale=np.full(8, 0.0234, np.float32))
    assert np.array_equal(one.k_pool, each.k_pool) and np.array_equal(one.v_pool, each.v_pool)
