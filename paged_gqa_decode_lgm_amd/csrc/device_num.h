// Device number formats and wave64 reductions for the lgm kernels (gfx950).
//
// bf16 and OCP E4M3 ("e4m3fn", the FP8 KV format named in the mainarch
// README's decode-attention section) conversions are written from the format
// definitions with integer arithmetic, so their rounding is exact by
// construction: round to nearest even, E4M3 saturating to +-448 and keeping
// the sign of zero (the static-FP8 KV write of the Loom Kernels README,
// "Position and KV", does not state its rounding; this is the reading taken).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lgm {

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------------ E4M3
// Exact decode: the 7 magnitude bits placed at fp32 bit 20 form an fp32 whose
// value is the E4M3 value times 2^-120 (normal codes get exponent E-127+... ,
// subnormal codes become fp32 subnormals M * 2^-129), so one exact multiply
// by 2^120 restores it.  0x7F/0xFF (NaN) are mapped to NaN explicitly.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t mag = c & 0x7fu;
  float v = __uint_as_float(((c & 0x80u) << 24) | (mag << 20)) * 0x1p120f;
  return mag == 0x7fu ? __uint_as_float(0x7fc00000u) : v;
}

// fp32 -> E4M3 byte: round to nearest even, |x| >= 448 saturates to 448,
// NaN -> 0x7F, zero keeps its sign.
__device__ __forceinline__ uint8_t f32_to_e4m3_rne_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                                   // NaN
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);                // >= 448 (and inf)
  if (a < 0x3c800000u) {                                               // < 2^-6: subnormal range
    // code = round-to-even(|x| * 2^9); |x| * 512 is exact
    const float m = rintf(__uint_as_float(a) * 512.0f);
    return (uint8_t)(sign | (uint32_t)m);                              // m == 8 is the smallest normal
  }
  // normal: keep 3 mantissa bits with round-to-nearest-even on fp32 bits,
  // then rebias the exponent (127 -> 7); a carry into the exponent is right.
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return (uint8_t)(sign | (code > 0x7eu ? 0x7eu : code));
}

// ------------------------------------------------------------------ wave64 reductions
// Sum / max over aligned groups of N lanes (N in 1, 2, 4, 8, 16, 32, 64).
// Within a 16-lane row the butterflies use DPP (quad_perm xor 1 / xor 2,
// row_half_mirror, row_mirror); wider groups use ds_swizzle-free shuffles.
// Every lane of a group ends with the bitwise identical result.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  if constexpr (N >= 4)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  if constexpr (N >= 8)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  if constexpr (N >= 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace lgm
