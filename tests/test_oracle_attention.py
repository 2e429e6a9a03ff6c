"""Pins for oracle.attention: closed forms, invariants, a library routine and
a hand-solved example (tests/golden/attention_tiny.txt)."""
import math

import numpy as np
import pytest
import torch

import workloads
from conftest import read_golden
from oracle import attention as A
from oracle import codecs


def _small(name="llama3_8b_gqa", **kw):
    base = dict(num_seqs=3, ctx=(1, 300), num_blocks=None)
    base.update(kw)
    return workloads.make_workload(workloads.CONFIGS[name].with_(**base))


def _q(w, seed=0):
    c = w.cfg
    return np.random.default_rng(seed).standard_normal((c.num_seqs, c.num_q_heads, c.head_dim))


def _pools(w):
    return workloads.storage_bits(w.k_pool), workloads.storage_bits(w.v_pool)


def _run(w, q, **kw):
    c = w.cfg
    kp, vp = _pools(w)
    ks = None if w.k_scale is None else w.k_scale.numpy()
    vs = None if w.v_scale is None else w.v_scale.numpy()
    if c.cache == "f32":
        kp, vp = w.k_pool.numpy(), w.v_pool.numpy()
    return A.paged_decode(q, kp, vp, w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale,
                          num_kv_heads=c.num_kv_heads, block_size=c.block_size, cache=c.cache,
                          k_scale=ks, v_scale=vs, **kw)


# ------------------------------------------------------------ closed forms
def test_golden_tiny_worked_example():
    g = {r[0].rstrip(":"): [float(v) for v in r[1:]] for r in read_golden("attention_tiny.txt")}
    q = np.array([g["q"]])
    K = np.array([g["k0"], g["k1"]])
    V = np.array([g["v0"], g["v1"]])
    out, lse, p = A.attend(q, K, V, 1.0)
    assert np.allclose(out[0], g["out"], atol=1e-14)
    assert math.isclose(lse[0], g["lse"][0], rel_tol=1e-14)
    assert np.allclose(p[0], [0.25, 0.75], atol=1e-15)
    # same example through the paged path: one block of size 2, split per token
    pool_k = np.zeros((3, 2, 1, 2), np.float32)
    pool_v = np.zeros((3, 2, 1, 2), np.float32)
    pool_k[2, :, 0] = K
    pool_v[2, :, 0] = V
    bt = np.array([[2]], np.int32)
    o2, l2 = A.paged_decode(q[None], pool_k, pool_v, bt, [2], 1.0, num_kv_heads=1, block_size=2, cache="f32")
    # fp32 storage of ln 3 perturbs the result by ~1e-8
    assert np.allclose(o2[0, 0], g["out"], atol=1e-6) and abs(l2[0, 0] - g["lse"][0]) < 1e-7
    o_p, lse_p, n = A.paged_decode_partials(q[None], pool_k, pool_v, bt, [2], 1.0, 1, num_kv_heads=1,
                                            block_size=2, cache="f32")
    assert n.tolist() == [2]
    assert np.allclose(o_p[0, 0, 0], g["v0"]) and np.allclose(o_p[0, 0, 1], g["v1"])
    m_out, m_lse = A.lse_merge(o_p, lse_p, n)
    assert np.allclose(m_out[0, 0], o2[0, 0], atol=1e-14) and abs(m_lse[0, 0] - l2[0, 0]) < 1e-14


def test_weights_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((777, 128)) * 3
    V = rng.standard_normal((777, 128))
    _, _, p = A.attend(q, K, V, 1 / math.sqrt(128))
    assert np.abs(p.sum(axis=1) - 1).max() <= 1e-12
    assert (p >= 0).all()


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    k = rng.standard_normal(64)
    K = np.tile(k, (50, 1))
    V = rng.standard_normal((50, 64))
    out, lse, _ = A.attend(rng.standard_normal((3, 64)), K, V, 0.125)
    assert np.abs(out - V.mean(axis=0)).max() <= 1e-12


def test_dominant_score_returns_its_value_row():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128)
    K = rng.standard_normal((200, 128)) * 0.1
    K[57] = 60.0 * q / (q @ q) * math.sqrt(128)  # score 60 vs ~|0.1|: gap >= 50
    V = rng.standard_normal((200, 128))
    out, _, _ = A.attend(q[None], K, V, 1 / math.sqrt(128))
    assert np.abs(out[0] - V[57]).max() <= 1e-15 * 200 + 1e-18 + np.exp(-50) * 10


def test_single_token_context_returns_v0_and_empty_context():
    w = _small(num_seqs=2, ctx=1)
    q = _q(w)
    out, lse = _run(w, q)
    kp, vp = _pools(w)
    for b in range(2):
        for h in range(32):
            v0 = A.gather_kv(vp, w.block_tables.numpy(), b, 1, h // 4, 16, "bf16")[0]
            assert np.array_equal(out[b, h], v0)
    w0 = _small(num_seqs=2, ctx=1)
    w0.context_lens[:] = torch.tensor([0, 1], dtype=torch.int32)
    out, lse = _run(w0, q)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


def test_matches_torch_sdpa_fp64_with_gqa():
    w = _small(num_seqs=3, ctx=(5, 200))
    c = w.cfg
    q = _q(w, 5)
    out, lse = _run(w, q)
    kp, vp = _pools(w)
    for b in range(c.num_seqs):
        L = int(w.context_lens[b])
        K = np.stack([A.gather_kv(kp, w.block_tables.numpy(), b, L, g, 16, "bf16") for g in range(8)])
        V = np.stack([A.gather_kv(vp, w.block_tables.numpy(), b, L, g, 16, "bf16") for g in range(8)])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b][:, None, :]), torch.from_numpy(K), torch.from_numpy(V),
            scale=c.softmax_scale, enable_gqa=True)[:, 0, :].numpy()
        assert np.abs(ref - out[b]).max() <= 1e-13


def test_identity_table_matches_dense_attention():
    """With the identity block table the paged cache is a dense [tokens, Hkv, D]
    array; attention over its first L rows (torch SDPA, no block-table
    gather) must equal the paged oracle.  Together with the block-shuffle
    invariance this pins the gather for any table."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, bs, NB = 3, 8, 2, 64, 16, 40
    kp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32)
    ctx = np.array([1, 17, 300], np.int32)
    q = rng.standard_normal((B, Hq, D))
    bt = np.tile(np.arange(NB, dtype=np.int32), (B, 1))
    o, _ = A.paged_decode(q, kp, vp, bt, ctx, 0.125, num_kv_heads=Hkv, block_size=bs, cache="f32")
    for b in range(B):
        dense_k = torch.from_numpy(kp.reshape(NB * bs, Hkv, D)[: ctx[b]].astype(np.float64)).permute(1, 0, 2)
        dense_v = torch.from_numpy(vp.reshape(NB * bs, Hkv, D)[: ctx[b]].astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b][:, None, :]), dense_k, dense_v, scale=0.125, enable_gqa=True)[:, 0].numpy()
        assert np.abs(ref - o[b]).max() <= 1e-13


# ------------------------------------------------------------ split-K / merge
@pytest.mark.parametrize("ps", [16, 512, 100000])
def test_split_equals_unsplit(ps):
    w = _small(num_seqs=4, ctx=(1, 1500))
    c = w.cfg
    q = _q(w, 6)
    out, lse = _run(w, q)
    kp, vp = _pools(w)
    o_p, lse_p, n = A.paged_decode_partials(q, kp, vp, w.block_tables.numpy(), w.context_lens.numpy(),
                                            c.softmax_scale, ps, num_kv_heads=8, block_size=16, cache="bf16")
    assert (n == -(-w.context_lens.numpy() // ps)).all()
    m_out, m_lse = A.lse_merge(o_p, lse_p, n)
    assert np.abs(m_out - out).max() <= 1e-12
    assert np.abs(m_lse - lse).max() <= 1e-12


def test_merge_identity_order_and_empty_partition():
    rng = np.random.default_rng(8)
    o = rng.standard_normal((2, 3, 5, 16))
    l = rng.standard_normal((2, 3, 5)) * 4
    one, one_l = A.lse_merge(o[:, :, :1], l[:, :, :1])
    assert np.array_equal(one, o[:, :, 0]) and np.allclose(one_l, l[:, :, 0], atol=0)
    perm = rng.permutation(5)
    a, al = A.lse_merge(o, l)
    b, bl = A.lse_merge(o[:, :, perm], l[:, :, perm])
    assert np.abs(a - b).max() <= 1e-14 and np.abs(al - bl).max() <= 1e-14
    l2 = l.copy()
    l2[:, :, 2] = -np.inf
    c, cl = A.lse_merge(o, l2)
    keep = [0, 1, 3, 4]
    d, dl = A.lse_merge(o[:, :, keep], l[:, :, keep])
    assert np.abs(c - d).max() <= 1e-14 and np.abs(cl - dl).max() <= 1e-14
    # an empty record weighs exactly zero whatever its row holds: memory
    # nobody wrote may be NaN or Inf
    o2 = o.copy()
    o2[0, :, 2] = np.nan
    o2[1, :, 2] = np.inf
    o2[1, 0, 2, ::2] = -np.inf
    c2, cl2 = A.lse_merge(o2, l2)
    assert np.array_equal(c2, c) and np.array_equal(cl2, cl)
    # all records empty: out = 0 and lse = -inf, even over NaN rows
    z, zl = A.lse_merge(np.full((1, 2, 3, 4), np.nan), np.full((1, 2, 3), -np.inf))
    assert np.array_equal(z, np.zeros((1, 2, 4))) and np.isneginf(zl).all()
    # counts limit each sequence to its first P_b records
    e, el = A.lse_merge(o, l, np.array([2, 5]))
    f, fl = A.lse_merge(o[:1, :, :2], l[:1, :, :2])
    assert np.array_equal(e[0], f[0]) and np.array_equal(el[0], fl[0])


def test_merge_closed_form_two_partitions():
    """Two partitions with lse a and b: weights e^a/(e^a+e^b), lse = log(e^a+e^b)."""
    o = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    l = np.array([[[math.log(2.0), math.log(6.0)]]])
    out, lse = A.lse_merge(o, l)
    assert np.allclose(out[0, 0], [0.25, 0.75], atol=1e-15)
    assert math.isclose(lse[0, 0], math.log(8.0), rel_tol=1e-15)


# ------------------------------------------------------------ paging / GQA
def test_block_shuffle_with_table_permutation_is_exact():
    w = _small(num_seqs=3, ctx=(30, 400))
    q = _q(w, 9)
    out, lse = _run(w, q)
    w2 = workloads.shuffled_copy(w, 123)
    assert not torch.equal(w2.block_tables, w.block_tables)
    out2, lse2 = _run(w2, q)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_poisoned_unused_slots_and_entries_change_nothing():
    w = _small(num_seqs=3, ctx=(20, 333))
    q = _q(w, 10)
    out, lse = _run(w, q)
    bt = w.block_tables.clone()
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    used = set()
    for b in range(3):
        L = int(w.context_lens[b])
        nb = -(-L // 16)
        used |= set(bt[b, :nb].tolist())
        bt[b, nb:] = torch.tensor([-7, 10 ** 9] * 600, dtype=torch.int32)[: bt.shape[1] - nb]
        last = int(bt[b, nb - 1])
        kp[last, L - (nb - 1) * 16:] = float("nan")   # slots past the context in the last block
        vp[last, L - (nb - 1) * 16:] = float("nan")
    unused = [i for i in range(kp.shape[0]) if i not in used]
    kp[unused] = float("nan")
    vp[unused] = float("nan")
    w2 = workloads.Workload(w.cfg, w.context_lens, bt, kp, vp, w.qkv, None, None)
    out2, lse2 = _run(w2, q)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_perturbing_one_kv_head_moves_only_its_query_group():
    w = _small(num_seqs=2, ctx=(50, 200))
    q = _q(w, 11)
    out, _ = _run(w, q)
    g = 5
    kp = w.k_pool.clone()
    kp[:, :, g, :] = kp[:, :, g, :] * 2
    out2, _ = _run(workloads.Workload(w.cfg, w.context_lens, w.block_tables, kp, w.v_pool, w.qkv, None, None), q)
    moved = np.abs(out2 - out).max(axis=(0, 2)) > 0
    assert moved.tolist() == [h // 4 == g for h in range(32)]


def test_perturbing_one_physical_block_moves_only_its_sequences():
    w = _small(num_seqs=4, ctx=(40, 300))
    q = _q(w, 12)
    out, _ = _run(w, q)
    pb = int(w.block_tables[2, 1])
    vp = w.v_pool.clone()
    vp[pb] = vp[pb] + 1
    out2, _ = _run(workloads.Workload(w.cfg, w.context_lens, w.block_tables, w.k_pool, vp, w.qkv, None, None), q)
    moved = np.abs(out2 - out).max(axis=(1, 2)) > 0
    assert moved.tolist() == [b == 2 for b in range(4)]


def test_fp8_dequant_applies_per_head_scales():
    """All K codes 0x38 (1.0) and V codes 0x40 (2.0): every key is equal, so the
    output is the common V row 2 * v_scale[g]."""
    w = _small("fp8_kv", num_seqs=2, ctx=(3, 40))
    kp = torch.full_like(w.k_pool.view(torch.uint8), 0x38).view(torch.float8_e4m3fn)
    vp = torch.full_like(w.v_pool.view(torch.uint8), 0x40).view(torch.float8_e4m3fn)
    w2 = workloads.Workload(w.cfg, w.context_lens, w.block_tables, kp, vp, w.qkv, w.k_scale, w.v_scale)
    out, _ = _run(w2, _q(w, 13))
    vs = w.v_scale.numpy().astype(np.float64)
    for h in range(32):
        assert np.allclose(out[:, h], 2.0 * vs[h // 4], rtol=0, atol=1e-15)
    assert codecs.e4m3_decode(np.array([0x40], np.uint8))[0] == 2.0


def _fp4_pool_to_f32_by_offsets(pool, bs, hkv, d):
    """Decode an FP4 pool byte by byte from the stated layout (codes of (t, g)
    at (t*Hkv + g)*D/2, two per byte, low nibble first; scales after all
    codes, one per 32 elements), without the oracle's views or dequantiser."""
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    nb = pool.shape[0]
    nc = bs * hkv * d // 2
    out = np.zeros((nb, bs, hkv, d), dtype=np.float32)
    for blk in range(nb):
        row = pool[blk]
        for t in range(bs):
            for g in range(hkv):
                base = (t * hkv + g) * d // 2
                sbase = nc + (t * hkv + g) * d // 32
                for e in range(d):
                    byte = int(row[base + e // 2])
                    code = byte & 0xF if e % 2 == 0 else byte >> 4
                    v = mag[code & 7] * (-1.0 if code & 8 else 1.0)
                    out[blk, t, g, e] = math.ldexp(v, int(row[sbase + e // 32]) - 127)
    return out


def test_fp4_cache_equals_f32_cache_of_its_decoded_values():
    """Attention over an FP4 pool equals attention over an fp32 pool holding
    the same values (every E2M1 value times a power of two is an fp32 value),
    decoded here from the layout's byte offsets alone."""
    w = _small("fp4_kv", num_seqs=2, ctx=(1, 90))
    c = w.cfg
    kp, vp = w.k_pool.numpy(), w.v_pool.numpy()
    kf = _fp4_pool_to_f32_by_offsets(kp, c.block_size, c.num_kv_heads, c.head_dim)
    vf = _fp4_pool_to_f32_by_offsets(vp, c.block_size, c.num_kv_heads, c.head_dim)
    q = _q(w, 21)
    args = (w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale)
    kw = dict(num_kv_heads=c.num_kv_heads, block_size=c.block_size)
    o4, l4 = A.paged_decode(q, kp, vp, *args, cache="fp4", **kw)
    o32, l32 = A.paged_decode(q, kf, vf, *args, cache="f32", **kw)
    assert np.array_equal(o4, o32) and np.array_equal(l4, l32)
    p4 = A.paged_decode_partials(q, kp, vp, *args, 32, cache="fp4", **kw)
    p32 = A.paged_decode_partials(q, kf, vf, *args, 32, cache="f32", **kw)
    assert all(np.array_equal(a, b) for a, b in zip(p4, p32))


# ------------------------------------------------------------------ cache views and scale granularity
def _to_hnd(pool):
    """NHD [NB, bs, Hkv, D] -> HND [NB, Hkv, bs, D], element by element."""
    nb, bs, hkv, d = pool.shape
    out = np.empty((nb, hkv, bs, d), dtype=pool.dtype)
    for blk in range(nb):
        for t in range(bs):
            for g in range(hkv):
                out[blk, g, t] = pool[blk, t, g]
    return out


def _fp4_to_hnd(pool, bs, hkv, d):
    """FP4 blocks with NHD parts -> the same blocks with head-major parts,
    byte by byte from the stated offsets."""
    nc = bs * hkv * d // 2
    out = np.empty_like(pool)
    for blk in range(pool.shape[0]):
        for t in range(bs):
            for g in range(hkv):
                src, dst = (t * hkv + g) * d // 2, (g * bs + t) * d // 2
                out[blk, dst:dst + d // 2] = pool[blk, src:src + d // 2]
                src, dst = nc + (t * hkv + g) * d // 32, nc + (g * bs + t) * d // 32
                out[blk, dst:dst + d // 32] = pool[blk, src:src + d // 32]
    return out


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "fp8_kv", "fp4_kv"])
def test_hnd_pool_equals_nhd_pool(name):
    """The same cache stored head-major inside each block gives bitwise the
    same attention, split or not."""
    w = _small(name, num_seqs=2, ctx=(1, 120))
    c = w.cfg
    kp, vp = _pools(w)
    if c.cache == "fp4":
        kh = _fp4_to_hnd(kp, c.block_size, c.num_kv_heads, c.head_dim)
        vh = _fp4_to_hnd(vp, c.block_size, c.num_kv_heads, c.head_dim)
    else:
        kh, vh = _to_hnd(kp), _to_hnd(vp)
    q = _q(w, 3)
    ks = None if w.k_scale is None else w.k_scale.numpy()
    vs = None if w.v_scale is None else w.v_scale.numpy()
    kw = dict(num_kv_heads=c.num_kv_heads, block_size=c.block_size, cache=c.cache, k_scale=ks, v_scale=vs)
    args = (w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale)
    a = A.paged_decode(q, kp, vp, *args, **kw)
    b = A.paged_decode(q, kh, vh, *args, layout="hnd", **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    pa = A.paged_decode_partials(q, kp, vp, *args, 32, **kw)
    pb = A.paged_decode_partials(q, kh, vh, *args, 32, layout="hnd", **kw)
    assert all(np.array_equal(x, y) for x, y in zip(pa, pb))


def test_per_tensor_fp8_scale_is_every_heads_scale():
    """A one-element scale array scales every kv head: the same as a per-head
    array holding that value for each head."""
    w = _small("fp8_kv", num_seqs=2, ctx=(5, 90))
    c = w.cfg
    kp, vp = _pools(w)
    q = _q(w, 4)
    args = (w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale)
    kw = dict(num_kv_heads=c.num_kv_heads, block_size=c.block_size, cache="fp8")
    one = A.paged_decode(q, kp, vp, *args, k_scale=np.array([0.013], np.float32),
                         v_scale=np.array([0.021], np.float32), **kw)
    each = A.paged_decode(q, kp, vp, *args, k_scale=np.full(8, 0.013, np.float32),
                          v_scale=np.full(8, 0.021, np.float32), **kw)
    assert np.array_equal(one[0], each[0]) and np.array_equal(one[1], each[1])
