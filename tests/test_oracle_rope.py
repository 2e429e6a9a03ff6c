"""Pins for oracle.rope: closed forms and invariants of the split-half rotation."""
import math

import numpy as np
import pytest

from oracle import rope

D = 128


def _x(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_inv_freq_closed_form():
    for theta in (1e4, 5e5, 1e6):
        w = rope.rope_inv_freq(theta, D)
        assert w[0] == 1.0
        assert math.isclose(w[D // 4], 1.0 / math.sqrt(theta), rel_tol=1e-14)   # theta^(-1/2)
        assert np.allclose(w[1:] / w[:-1], theta ** (-2.0 / D), rtol=1e-13)


def test_position_zero_is_identity():
    x = _x((5, D))
    assert np.array_equal(rope.rope_neox_f64(x, 0, 1e4), x)
    x32 = x.astype(np.float32)
    assert np.array_equal(rope.rope_neox_f32_recipe(x32, 0, 1e4), x32)


def test_first_pair_angle_is_position_in_radians():
    """Pair 0 has w_0 = 1: (x0, x_{D/2}) rotates by exactly pos radians."""
    x = np.zeros(D)
    x[0] = 1.0
    for pos in (1, 7, 255, 131071):
        y = rope.rope_neox_f64(x, pos, 5e5)
        assert math.isclose(y[0], math.cos(pos), abs_tol=1e-15)
        assert math.isclose(y[D // 2], math.sin(pos), abs_tol=1e-15)


def test_split_half_pairing_one_hot():
    """Basis vector e_j only mixes with e_{j +- D/2} (split-half, not adjacent pairs)."""
    for j in (0, 3, D // 2 - 1, D // 2, D - 1):
        x = np.zeros(D)
        x[j] = 1.0
        y = rope.rope_neox_f64(x, 37, 1e4)
        partner = (j + D // 2) % D
        nz = set(np.flatnonzero(np.abs(y) > 1e-300).tolist())
        assert nz <= {j, partner}
        i = j % (D // 2)
        ang = 37 * rope.rope_inv_freq(1e4, D)[i]
        sign = 1.0 if j >= D // 2 else -1.0      # lo half: -x_hi*s ; hi half: +x_lo*s
        assert math.isclose(y[j], math.cos(ang), abs_tol=1e-15)
        assert math.isclose(y[partner], -sign * math.sin(ang), abs_tol=1e-15)


def test_pair_norms_preserved():
    x = _x((4, 6, D), 1)
    y = rope.rope_neox_f64(x, np.array([1, 100, 5000, 131071]), 1e6)
    h = D // 2
    n_in = x[..., :h] ** 2 + x[..., h:] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:] ** 2
    assert np.abs(n_in - n_out).max() <= 1e-12 * max(1.0, n_in.max())


def test_composition():
    x = _x((3, D), 2)
    for a, b in ((3, 5), (1000, 24), (65536, 65535)):
        y = rope.rope_neox_f64(rope.rope_neox_f64(x, a, 5e5), b, 5e5)
        z = rope.rope_neox_f64(x, a + b, 5e5)
        assert np.abs(y - z).max() <= 1e-9


def test_relative_position_property():
    """<R(p) q, R(p') k> depends only on p - p'."""
    q, k = _x(D, 3), _x(D, 4)
    for delta in (0, 1, 17, 4095):
        ref = None
        for p0 in (0, 100, 9999, 131072 - delta - 1):
            v = rope.rope_neox_f64(q, p0 + delta, 1e4) @ rope.rope_neox_f64(k, p0, 1e4)
            ref = v if ref is None else ref
            assert abs(v - ref) <= 1e-9 * max(1.0, abs(ref))


def test_per_row_positions():
    x = _x((3, 2, D), 5)
    pos = np.array([0, 9, 300])
    y = rope.rope_neox_f64(x, pos, 1e4)
    for b in range(3):
        assert np.array_equal(y[b], rope.rope_neox_f64(x[b], int(pos[b]), 1e4))


def test_f32_recipe_close_to_exact():
    """The fp32 recipe stays within a few fp32 ulps of the exact rotation:
    two rounded products and one rounded sum, with cos/sin off by <= 1/2 ulp."""
    x32 = _x((64, D), 6).astype(np.float32)
    pos = np.arange(64) * 2047
    y = rope.rope_neox_f32_recipe(x32, pos, 1e6).astype(np.float64)
    z = rope.rope_neox_f64(x32.astype(np.float64), pos, 1e6)
    h = D // 2
    scale = np.abs(np.concatenate([x32[:, :h], x32[:, :h]], 1)) + np.abs(np.concatenate([x32[:, h:], x32[:, h:]], 1))
    assert (np.abs(y - z) <= 4 * 2.0 ** -24 * scale + 1e-30).all()


def test_f32_recipe_exact_values_small_case():
    """pos 1, D = 2, theta irrelevant (w_0 = 1): each step rounded to fp32."""
    x = np.array([[1.5, -0.25]], np.float32)
    c, s = np.float32(math.cos(1.0)), np.float32(math.sin(1.0))
    want = np.array([[np.float32(np.float32(1.5 * c) - np.float32(-0.25 * s)),
                      np.float32(np.float32(-0.25 * c) + np.float32(1.5 * s))]], np.float32)
    got = rope.rope_neox_f32_recipe(x, 1, 1e4)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ interleaved (GPT-J) pairs
def test_interleaved_is_neox_of_the_even_odd_split():
    """Moving the even elements to the first half and the odd ones to the
    second turns adjacent pairs (2i, 2i+1) into split-half pairs (i, i+D/2)
    with the same frequency index: both rotations must agree bit for bit."""
    x = _x((3, 4, D), 7)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    pos = np.array([0, 9, 4097])
    for theta in (1e4, 5e5):
        a = rope.rope_interleaved_f64(x, pos, theta)
        b = rope.rope_neox_f64(x[..., perm], pos, theta)[..., inv]
        assert np.array_equal(a, b)
        x32 = x.astype(np.float32)
        a32 = rope.rope_interleaved_f32_recipe(x32, pos, theta)
        b32 = rope.rope_neox_f32_recipe(x32[..., perm], pos, theta)[..., inv]
        assert np.array_equal(a32, b32)


def test_interleaved_first_pair_and_identity():
    x = np.zeros(D)
    x[0] = 1.0
    for pos in (1, 7, 255):
        y = rope.rope_interleaved_f64(x, pos, 1e6)
        assert math.isclose(y[0], math.cos(pos), abs_tol=1e-15)
        assert math.isclose(y[1], math.sin(pos), abs_tol=1e-15)
        assert np.count_nonzero(y) == 2
    z = _x((2, D))
    assert np.array_equal(rope.rope_interleaved_f64(z, 0, 1e4), z)


def test_interleaved_relative_position():
    """<R(p) q, R(p') k> depends only on p - p'."""
    q, k = _x(D, 1), _x(D, 2)
    ref = rope.rope_interleaved_f64(q, 40, 1e4) @ rope.rope_interleaved_f64(k, 30, 1e4)
    for p in (10, 1000, 77777):
        v = rope.rope_interleaved_f64(q, p + 10, 1e4) @ rope.rope_interleaved_f64(k, p, 1e4)
        assert math.isclose(v, ref, rel_tol=1e-9, abs_tol=1e-9)
