"""Pins for oracle.codecs: hand-derived fixtures, library casts, brute force."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import codecs


def _f(s):
    return float.fromhex(s) if s.lower().startswith(("0x", "-0x")) else float(s)


# ------------------------------------------------------------------ E4M3
def test_e4m3_golden_cases():
    for val, code, *_ in read_golden("e4m3_cases.txt"):
        x = np.float32(_f(val))
        got = int(codecs.e4m3_encode(np.array([x]))[0])
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_nan_code():
    assert int(codecs.e4m3_encode(np.array([np.nan]))[0]) == 0x7F
    assert np.isnan(codecs.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_decode_closed_form_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # closed-form spot values: extremes of each range
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x80] == 0.0 and np.signbit(ours[0x80])


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = codecs.e4m3_encode(codecs.e4m3_decode(codes))
    assert (back == codes).all()


def test_e4m3_encode_vs_torch_cast_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(50),
        rng.uniform(-448, 448, 200_000).astype(np.float32),
        (rng.standard_normal(100_000) * 1e-3).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = codecs.e4m3_encode(x)
    assert (ours == ref).all()


def test_e4m3_every_midpoint_and_neighbours_brute_force():
    """At each midpoint between adjacent codes the even code wins; one fp32
    ulp either side picks the nearer code.  Checked against brute-force
    nearest-value search written independently below."""
    vals = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    xs = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    xs = np.concatenate([xs, -xs])
    ours = codecs.e4m3_encode(xs)
    for x, c in zip(xs, ours):
        a = abs(float(x))
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
        want |= 0x80 if np.signbit(x) else 0
        assert int(c) == int(want), (float(x), hex(int(c)), hex(int(want)))


def test_e4m3_dense_sweep_brute_force():
    xs = np.linspace(-470, 470, 40001, dtype=np.float32)
    vals = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    ours = codecs.e4m3_encode(xs)
    for x, c in zip(xs[::7], ours[::7]):
        a = min(abs(float(x)), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
        want |= 0x80 if np.signbit(x) else 0
        assert int(c) == int(want)


def test_e4m3_saturation_and_signed_zero():
    x = np.array([448.0, 449.0, 464.0, 1e30, np.inf, -449.0, -np.inf, -1e-30, 1e-30, -0.0], np.float64)
    got = codecs.e4m3_encode(x).tolist()
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00, 0x80]


# ------------------------------------------------------------------ bf16
def test_bf16_golden_cases():
    for val, bits, *_ in read_golden("bf16_cases.txt"):
        x = np.float32(_f(val))
        assert float(x) == _f(val), "fixture value must be exact in fp32"
        got = int(codecs.bf16_encode(np.array([x]))[0])
        assert got == int(bits, 16), (val, hex(got), bits)


def test_bf16_vs_torch_random_patterns_and_ties():
    rng = np.random.default_rng(11)
    pats = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = pats.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < np.float32(3.3e38))]
    # every tie: low 16 bits exactly 0x8000, both parities of bit 16
    ties = (rng.integers(0, 2 ** 15, 1 << 16, dtype=np.uint64).astype(np.uint32) << np.uint32(17)) | np.uint32(0x8000)
    ties = np.concatenate([ties, ties | np.uint32(1 << 16)]).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < np.float32(3.3e38))]
    for arr in (x, ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (codecs.bf16_encode(arr) == ref).all()


def test_bf16_decode_exact():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = codecs.bf16_decode(bits)
    assert ((ours == ref) | (np.isnan(ours) & np.isnan(ref))).all()
