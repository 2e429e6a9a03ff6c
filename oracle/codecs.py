"""Storage codecs, written from the number formats' definitions (oracle only).

bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits; a value
is rounded to the nearest representable one, ties to the even mantissa.  The
bf16 KV storage with fp32 accumulation the oracle mirrors is the one in
microLLM-rocm's ledger ("opt-in BF16 KV Storage ... FP32 Attention
accumulation").

E4M3: the OCP 8-bit float "e4m3fn" that mainarch's decode-attention section
names as its FP8 KV format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits, no infinities, only S.1111.111 is NaN, so the largest finite magnitude
is 1.75 * 2**8 = 448 and the smallest subnormal is 2**-9.  Loom Kernels'
FP8 KV write quantises with static scales; the pages give no rounding or
overflow rule, so the oracle takes round-to-nearest-even with saturation to
+-448 and keeps the sign of values that round to zero.

The encoder here deliberately works by nearest-neighbour search over the
decoded code table rather than by bit manipulation.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


# ----------------------------------------------------------------- bf16
def bf16_round(x) -> np.ndarray:
    """Round (float64 view of) x to the nearest bf16 value, ties to even.

    For finite nonzero x with binary exponent e (2**e <= |x| < 2**(e+1)) the
    bf16 spacing is 2**(e-7) (normal range) or 2**-133 (subnormal range);
    x / spacing is rounded to an integer with ties to even (np.rint)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        xf = x[fin]
        _, e2 = np.frexp(xf)  # xf = m * 2**e2, 0.5 <= |m| < 1  =>  e = e2 - 1
        e = e2.astype(np.int64) - 1
        e = np.maximum(e, -126)  # below the normal range the spacing is fixed
        spacing = np.ldexp(1.0, (e - 7).astype(np.int32))
        r = np.rint(xf / spacing) * spacing
        r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, xf), r)
        out[fin] = r
    return out


def bf16_bits_from_value(v) -> np.ndarray:
    """Bit pattern of values that are already exactly representable in bf16."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_encode(x) -> np.ndarray:
    """x (any float) -> bf16 bits, round to nearest even."""
    return bf16_bits_from_value(bf16_round(x))


def bf16_decode(bits) -> np.ndarray:
    """bf16 bits -> float64 value (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------- E4M3
def e4m3_decode(codes) -> np.ndarray:
    """E4M3 (e4m3fn) byte -> float64, from the field definition:
    exponent field E, mantissa field M: E == 0 -> M * 2**-9 (subnormal),
    otherwise (1 + M/8) * 2**(E-7); 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.power(2.0, E - 7))
    mag = np.where((E == 0xF) & (M == 0x7), np.nan, mag)
    return sign * mag


_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: all finite non-negative
_POS_VALUES = e4m3_decode(_POS_CODES)                   # strictly increasing


def e4m3_encode(x) -> np.ndarray:
    """float -> E4M3 byte: nearest finite code, ties to the even code,
    magnitudes beyond 448 saturate to +-448, NaN -> 0x7F, sign kept for zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    a_c = np.minimum(np.where(np.isnan(a), 0.0, a), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a_c, side="left")        # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo = a_c - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a_c == _POS_VALUES[hi], _POS_CODES[hi], code).astype(np.uint8)
    code = code | np.where(neg, np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    code = np.where(np.isnan(a), np.uint8(E4M3_NAN), code).astype(np.uint8)
    return code
