"""Planted mistakes in the oracle (on the CPU only): each plausible slip — a
dropped term, a wrong sign or index, a transposed operand — must make at least
one of the pins in test_oracle_*.py fail."""
import numpy as np
import pytest

import test_oracle_append as T_AP
import test_oracle_attention as T_A
import test_oracle_codecs as T_C
import test_oracle_rope as T_R
from oracle import append as AP
from oracle import attention as A
from oracle import codecs, rope


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_rope_wrong_sign_is_caught(monkeypatch):
    def bad(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        h = x.shape[-1] // 2
        ang = rope._per_row(rope.rope_angles(pos, theta, x.shape[-1]), x.ndim)
        c, s = np.cos(ang), np.sin(ang)
        return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], -1)
    monkeypatch.setattr(rope, "rope_neox_f64", bad)
    _fails(T_R.test_pair_norms_preserved)


def test_rope_adjacent_pairs_instead_of_split_half_is_caught(monkeypatch):
    def bad(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        ang = rope._per_row(rope.rope_angles(pos, theta, D), x.ndim)
        c, s = np.cos(ang), np.sin(ang)
        ev, od = x[..., 0::2], x[..., 1::2]
        y = np.empty_like(x)
        y[..., 0::2] = ev * c - od * s
        y[..., 1::2] = od * c + ev * s
        return y
    monkeypatch.setattr(rope, "rope_neox_f64", bad)
    _fails(T_R.test_split_half_pairing_one_hot)


def test_rope_dropped_factor_two_in_frequency_is_caught(monkeypatch):
    monkeypatch.setattr(rope, "rope_inv_freq",
                        lambda theta, D: np.power(float(theta), -np.arange(D // 2) / D))
    _fails(T_R.test_inv_freq_closed_form)


def test_attention_dropped_scale_is_caught(monkeypatch):
    orig = A.attend
    monkeypatch.setattr(A, "attend", lambda q, K, V, scale: orig(q, K, V, 1.0))
    _fails(T_A.test_matches_torch_sdpa_fp64_with_gqa)


def test_attention_transposed_value_use_is_caught(monkeypatch):
    def bad(q, K, V, scale):
        q = np.asarray(q, dtype=np.float64)
        s = scale * (q @ K.T)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out = (p @ K)  # keys used as values
        return out, np.log(np.exp(s).sum(1)), p
    monkeypatch.setattr(A, "attend", bad)
    _fails(T_A.test_golden_tiny_worked_example)


def test_interleaved_gqa_head_mapping_is_caught(monkeypatch):
    def bad(q, k_pool, v_pool, block_tables, context_lens, softmax_scale, *, num_kv_heads, block_size,
            cache, k_scale=None, v_scale=None, seqs=None):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, D = q.shape
        out = np.zeros((B, Hq, D))
        lse = np.zeros((B, Hq))
        for b in range(B):
            L = int(context_lens[b])
            for h in range(Hq):
                g = h % num_kv_heads
                K = A.gather_kv(k_pool, block_tables, b, L, g, block_size, cache, k_scale)
                V = A.gather_kv(v_pool, block_tables, b, L, g, block_size, cache, v_scale)
                o, l, _ = A.attend(q[b, h:h + 1], K, V, softmax_scale)
                out[b, h], lse[b, h] = o[0], l[0]
        return out, lse
    monkeypatch.setattr(A, "paged_decode", bad)
    _fails(T_A.test_perturbing_one_kv_head_moves_only_its_query_group)


def test_off_by_one_block_index_is_caught(monkeypatch):
    orig = A.gather_kv
    def bad(pool, block_tables, b, L, g, block_size, cache, scale=None):
        if L <= 0:
            return orig(pool, block_tables, b, L, g, block_size, cache, scale)
        j = np.arange(L)
        pb = np.asarray(block_tables)[b, (j + 1) // block_size].astype(np.int64)  # slip
        raw = np.asarray(pool)[pb, j % block_size, g, :]
        return A.decode_rows(raw, cache, None if scale is None else float(scale[g]))
    monkeypatch.setattr(A, "gather_kv", bad)
    _fails(T_A.test_identity_table_matches_dense_attention)


def test_merge_without_normalisation_is_caught(monkeypatch):
    def bad(o_p, lse_p, num_parts=None):
        o_p, lse_p = np.asarray(o_p), np.asarray(lse_p)
        M = lse_p.max(axis=2, keepdims=True)
        w = np.exp(lse_p - M)
        return (w[..., None] * o_p).sum(2), (M[..., 0] + np.log(w.sum(2)))
    monkeypatch.setattr(A, "lse_merge", bad)
    _fails(T_A.test_merge_closed_form_two_partitions)


def test_merge_reading_empty_rows_is_caught(monkeypatch):
    def bad(o_p, lse_p, num_parts=None):
        o_p, lse_p = np.asarray(o_p, np.float64), np.asarray(lse_p, np.float64)
        B, H, P, D = o_p.shape
        out, lse = np.zeros((B, H, D)), np.full((B, H), -np.inf)
        for b in range(B):
            n = P if num_parts is None else int(num_parts[b])
            for h in range(H):
                ls = lse_p[b, h, :n]
                if n == 0 or not np.isfinite(ls).any():
                    continue
                w = np.exp(ls - ls.max())  # 0 for an empty record, then 0 * NaN = NaN
                out[b, h] = (w[:, None] * o_p[b, h, :n]).sum(0) / w.sum()
                lse[b, h] = ls.max() + np.log(w.sum())
        return out, lse
    monkeypatch.setattr(A, "lse_merge", bad)
    _fails(T_A.test_merge_identity_order_and_empty_partition)


def test_append_at_wrong_position_is_caught(monkeypatch):
    orig = AP.rope_kv_append
    def bad(qkv, context_lens, *a, **k):
        return orig(qkv, np.asarray(context_lens) - 1, *a, **k)  # writes at ctx - 2
    monkeypatch.setattr(AP, "rope_kv_append", bad)
    _fails(T_AP.test_only_target_slots_change, "qwen2.5_1.5b_gqa")


def test_e4m3_ties_away_from_zero_is_caught(monkeypatch):
    vals = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.minimum(np.abs(x), 448.0)
        d = np.abs(vals[None, :] - a[:, None])
        best = np.argmin(d - 1e-12 * np.arange(0x7F)[None, :], axis=1)  # ties go up
        return (best | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(codecs, "e4m3_encode", bad)
    _fails(T_C.test_e4m3_golden_cases)


def test_e4m3_missing_saturation_is_caught(monkeypatch):
    orig = codecs.e4m3_encode
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        return np.where(np.abs(x) > 464, np.uint8(0x7F), orig(x)).astype(np.uint8)
    monkeypatch.setattr(codecs, "e4m3_encode", bad)
    _fails(T_C.test_e4m3_saturation_and_signed_zero)


def test_bf16_truncation_instead_of_rounding_is_caught(monkeypatch):
    def bad(x):
        v = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(codecs, "bf16_encode", bad)
    _fails(T_C.test_bf16_golden_cases)


def test_e2m1_ties_away_from_zero_is_caught(monkeypatch):
    orig = codecs.e2m1_encode
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        spacing = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
        up = np.floor(a / spacing + 0.5) * spacing  # ties away from zero
        return orig(np.copysign(np.minimum(up, 6.0), x))
    monkeypatch.setattr(codecs, "e2m1_encode", bad)
    _fails(T_C.test_e2m1_golden_cases)


def test_mx_scale_exponent_off_by_one_is_caught(monkeypatch):
    orig = codecs.mx_block_exponent
    monkeypatch.setattr(codecs, "mx_block_exponent", lambda amax: orig(amax) + 1)
    _fails(T_C.test_mx_golden_blocks)
    _fails(T_C.test_mx_scale_rule_invariants)


def test_fp4_swapped_nibbles_are_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes, dtype=np.uint8)
        return (c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)
    monkeypatch.setattr(codecs, "fp4_pack", bad)
    _fails(T_C.test_mx_golden_blocks)


def test_fp4_scales_before_codes_is_caught(monkeypatch):
    def bad(pool, block_size, num_kv_heads, head_dim, layout="nhd"):
        p = np.asarray(pool, dtype=np.uint8)
        ns = block_size * num_kv_heads * head_dim // 32
        return (p[:, ns:].reshape(p.shape[0], block_size, num_kv_heads, head_dim // 2),
                p[:, :ns].reshape(p.shape[0], block_size, num_kv_heads, head_dim // 32))
    monkeypatch.setattr(codecs, "fp4_block_views", bad)
    _fails(T_C.test_fp4_block_views_address_the_stated_bytes)
    _fails(T_A.test_fp4_cache_equals_f32_cache_of_its_decoded_values)


def test_fp4_scale_per_16_elements_is_caught(monkeypatch):
    def bad(packed, scales):
        v = codecs.e2m1_decode(codecs.fp4_unpack(packed))
        s = codecs.e8m0_decode(scales)
        idx = (np.arange(v.shape[-1]) // 16) % s.shape[-1]
        return v * s[..., idx]
    monkeypatch.setattr(codecs, "mx_fp4_dequantize", bad)
    _fails(T_A.test_fp4_cache_equals_f32_cache_of_its_decoded_values)


def test_interleaved_with_split_half_pairs_is_caught(monkeypatch):
    monkeypatch.setattr(rope, "rope_interleaved_f64", rope.rope_neox_f64)
    _fails(T_R.test_interleaved_is_neox_of_the_even_odd_split)
    _fails(T_R.test_interleaved_first_pair_and_identity)


def test_interleaved_with_doubled_frequency_index_is_caught(monkeypatch):
    def bad(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        ang = rope._per_row(np.asarray(pos, np.float64)[..., None] * np.power(theta, -4.0 * np.arange(D // 2) / D),
                            x.ndim)
        c, s = np.cos(ang), np.sin(ang)
        y = np.empty_like(x)
        y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
        return y
    monkeypatch.setattr(rope, "rope_interleaved_f64", bad)
    _fails(T_R.test_interleaved_is_neox_of_the_even_odd_split)


def test_hnd_view_without_the_axis_swap_is_caught(monkeypatch):
    orig = A.kv_source
    def bad(pool, cache, block_size, num_kv_heads, head_dim, layout="nhd"):
        if layout == "hnd" and cache != "fp4":
            return np.asarray(pool).reshape(pool.shape[0], block_size, num_kv_heads, head_dim)
        return orig(pool, cache, block_size, num_kv_heads, head_dim, layout)
    monkeypatch.setattr(A, "kv_source", bad)
    _fails(T_A.test_hnd_pool_equals_nhd_pool, "llama3_8b_gqa")


def test_per_tensor_scale_read_as_one_is_caught(monkeypatch):
    orig = A.gather_kv
    def bad(pool, block_tables, b, L, g, block_size, cache, scale=None):
        if scale is not None and np.asarray(scale).size == 1:
            scale = np.ones(64, np.float32)  # the one-element array taken as "no scale"
        return orig(pool, block_tables, b, L, g, block_size, cache, scale)
    monkeypatch.setattr(A, "gather_kv", bad)
    _fails(T_A.test_per_tensor_fp8_scale_is_every_heads_scale)


def test_mla_dropped_positional_term_is_caught(monkeypatch):
    import test_oracle_mla as T_M
    from oracle import mla as M
    def bad(q_lat, q_pe, c, r, scale):
        return orig(q_lat, np.zeros_like(np.asarray(q_pe, dtype=np.float64)), c, r, scale)
    orig = M.mla_attend
    monkeypatch.setattr(M, "mla_attend", bad)
    _fails(T_M.test_matches_torch_sdpa_fp64)


def test_mla_value_from_positional_rows_is_caught(monkeypatch):
    import test_oracle_mla as T_M
    from oracle import mla as M
    def bad(q_lat, q_pe, c, r, scale):
        o, l = orig(q_lat, q_pe, c, r, scale)
        return o * 0.5, l   # a mis-scaled value path
    orig = M.mla_attend
    monkeypatch.setattr(M, "mla_attend", bad)
    _fails(T_M.test_matches_torch_sdpa_fp64)
    _fails(T_M.test_equal_latent_rows_return_that_row_and_empty_context)
