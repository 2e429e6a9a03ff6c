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


# ----------------------------------------------------------------- MX FP4: E2M1 codes with E8M0 block scales
# mainarch's decode-attention section stores KV as 4-bit E2M1 values with
# E8M0 block scales (dequantised through the hardware's scaled FP4
# conversion).  The pages give neither the block size nor the scale rule; the
# oracle takes the OCP Microscaling (MX) v1.0 definitions, where those names
# come from:
#   E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no infinities
#         and no NaN: E == 0 -> M * 0.5 (subnormal), else (1 + M/2) * 2**(E-1);
#         the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
#   E8M0: an unbiased-exponent byte, value 2**(byte - 127); 0xFF is NaN.
#   Block: 32 consecutive elements share one scale X = 2**(floor(log2(amax)) - 2),
#         2 being the exponent of E2M1's largest normal (6 = 1.5 * 2**2);
#         elements are V_i / X rounded to nearest E2M1, ties to the even
#         mantissa, magnitudes above 6 saturating to 6.
# Readings where MX leaves a choice: an all-zero block takes the smallest
# scale (byte 0x00); the exponent is clamped to E8M0's [-127, 127]; values
# that round to zero keep their sign (code 0x8 for negative ones), as for FP8.
# Packing: element 2i sits in the low nibble of byte i, element 2i+1 in the
# high nibble.

MX_BLOCK = 32
E2M1_MAX = 6.0
E2M1_EMAX = 2
E8M0_BIAS = 127
E8M0_NAN = 0xFF


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (low 4 bits) -> float64, from the field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    M = c & 0x1
    mag = np.where(E == 0, M * 0.5, (1.0 + M / 2.0) * np.power(2.0, E - 1))
    return sign * mag


def e8m0_decode(b) -> np.ndarray:
    """E8M0 byte -> float64 scale 2**(b - 127); 0xFF is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == E8M0_NAN, np.nan, np.ldexp(1.0, (b - E8M0_BIAS).astype(np.int32)))


def e2m1_encode(x) -> np.ndarray:
    """float (already divided by the block scale) -> E2M1 code.

    Rounds |x| in its own binade: the spacing is 0.5 below 2 (E2M1's subnormal
    step and the first normal binade share it), 1 in [2, 4) and 2 in [4, 8);
    |x| / spacing goes to the nearest integer with ties to even, which is the
    even mantissa.  Magnitudes that round above 6 saturate to 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.isnan(a).any():
        raise ValueError("E2M1 has no NaN")
    spacing = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / spacing) * spacing, E2M1_MAX)  # rint: ties to even multiple of the spacing
    # value -> code: exponent field and mantissa bit of the rounded magnitude
    E = np.where(r < 1.0, 0, np.floor(np.log2(np.maximum(r, 1.0))).astype(np.int64) + 1)
    M = np.where(E == 0, (r / 0.5).astype(np.int64), (r / np.ldexp(1.0, (E - 1).astype(np.int32)) - 1.0) * 2.0)
    code = (E.astype(np.int64) << 1) | M.astype(np.int64)
    code = code | np.where(np.signbit(x), 0x8, 0)
    return code.astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent of blocks with absolute maxima amax: floor(log2 amax) - 2,
    clamped to [-127, 127]; an all-zero block gets -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = m * 2**e2, 0.5 <= m < 1
    e = e2.astype(np.int64) - 1 - E2M1_EMAX
    e = np.where(amax > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def mx_fp4_quantize(x):
    """Rows x [..., D] (D a multiple of 32) -> (codes uint8 [..., D], one code
    per element, and scale bytes uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    e = mx_block_exponent(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.ldexp(1.0, e.astype(np.int32))[..., None]  # a power of two: exact
    codes = e2m1_encode(scaled).reshape(x.shape)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def fp4_pack(codes) -> np.ndarray:
    """Codes [..., D] -> bytes [..., D/2]: element 2i low nibble, 2i+1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def fp4_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mx_fp4_dequantize(packed, scales) -> np.ndarray:
    """Packed codes [..., D/2] and scale bytes [..., D/32] -> float64 [..., D] (exact)."""
    v = e2m1_decode(fp4_unpack(packed))
    s = e8m0_decode(scales)
    D = v.shape[-1]
    return (v.reshape(v.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)) * s[..., None]).reshape(v.shape)


def fp4_block_views(pool, block_size: int, num_kv_heads: int, head_dim: int, layout: str = "nhd"):
    """An FP4 cache pool, uint8 [num_blocks, block_bytes], as its two parts.

    Each block holds its codes, NHD [block_size][num_kv_heads][head_dim/2]
    bytes (HND: [num_kv_heads][block_size][head_dim/2]), followed by its
    scales in the same order with head_dim/32 bytes per row.  Returns
    (codes [NB, bs, Hkv, D/2], scales [NB, bs, Hkv, D/32]), views into the
    pool whatever the stored order."""
    p = np.asarray(pool, dtype=np.uint8)
    nb = p.shape[0]
    nc = block_size * num_kv_heads * head_dim // 2
    ns = block_size * num_kv_heads * head_dim // MX_BLOCK
    if p.shape[1] != nc + ns:
        raise ValueError(f"FP4 block holds {nc + ns} bytes, pool rows have {p.shape[1]}")
    if layout == "nhd":
        return (p[:, :nc].reshape(nb, block_size, num_kv_heads, head_dim // 2),
                p[:, nc:].reshape(nb, block_size, num_kv_heads, head_dim // MX_BLOCK))
    if layout == "hnd":
        return (np.swapaxes(p[:, :nc].reshape(nb, num_kv_heads, block_size, head_dim // 2), 1, 2),
                np.swapaxes(p[:, nc:].reshape(nb, num_kv_heads, block_size, head_dim // MX_BLOCK), 1, 2))
    raise ValueError(layout)


def fp4_block_bytes(block_size: int, num_kv_heads: int, head_dim: int) -> int:
    return block_size * num_kv_heads * (head_dim // 2 + head_dim // MX_BLOCK)
