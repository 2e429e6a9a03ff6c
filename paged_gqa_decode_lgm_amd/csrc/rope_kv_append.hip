// Fused NeoX RoPE + paged-KV append of the new token (Loom Kernels README,
// "Supported operator paths", row "Position and KV": packed QKV in, rotated
// Q out, K/V written into NHD cache blocks natively or as static-scaled FP8
// E4M3; "Next value program": exact E4M3 bytes; microLLM-rocm ledger:
// split-half RoPE, positions-aware RoPE with a mapped KV store).
//
// One workgroup per sequence.  The D/2 rotation factors for the sequence's
// position are computed once into LDS: angle = pos * theta^(-2i/D) with
// theta^(-2i/D), the angle, its cosine and sine in fp64, cosine and sine
// rounded once to fp32.  The rotation itself is fp32 with every product and
// sum rounded on its own: this translation unit is built with
// -ffp-contract=off and the pragma below, so no multiply-add is fused.
// Rows move as eight-element vectors whenever the pointers and the QKV row
// stride allow it.  Contract variants (Loom, "Position and KV" row):
// LGM_ROPE_INTERLEAVED rotates adjacent pairs (x[2i], x[2i+1]) with the same
// angles and the same fp32 operations; LGM_CACHE_HND stores each block
// head-major; LGM_SCALE_PER_TENSOR uses one FP8 scale for every kv head.
//
// FP4 caches (mainarch README, decode-attention section: E2M1 KV with E8M0
// block scales; OCP MX block rule, as the library header states): eight
// lanes per 32-element block of a new K or V row.  They evaluate the block's
// rotated values with the same fp32 operations as the Q path, take the
// block's largest magnitude, the scale exponent X = floor(log2 amax) - 2
// (exact, from ilogbf), multiply by 2^-X (exact: a power of two), and round
// each value to E2M1 by comparing its magnitude with the midpoints of the
// code values (ties go to the even mantissa, magnitudes above 5 go to 6).
#include "device_num.h"
#include "lgm_internal.h"

#pragma clang fp contract(off)

namespace lgm {
namespace {

// One workgroup per sequence.  512 threads take a 32/8-head row's Q and K
// chunks and its V vectors in one pass each (256 needed a second pass for
// the K chunks): bf16 append 5.5 -> 4.8 us, FP8 7.6 -> 6.1 us on 64 and
// 128 sequences.
constexpr int kThreads = 512;
constexpr int kMaxHalf = 128;

// Eight consecutive elements of a dtype (one 16-byte load for bf16, two for fp32).
template <class T>
struct alignas(8 * sizeof(T)) Vec8 {
  T v[8];
};

struct ActF32 {
  using elem_t = float;
  __device__ static float load(const elem_t* p) { return *p; }
  __device__ static elem_t store(float x) { return x; }
};
struct ActBF16 {
  using elem_t = uint16_t;
  __device__ static float load(const elem_t* p) { return bf16_to_f32(*p); }
  __device__ static elem_t store(float x) { return f32_to_bf16_rne(x); }
};
struct CacheF32 {
  static constexpr bool kFp4 = false;
  using elem_t = float;
  __device__ static elem_t store(float x, float) { return x; }
};
struct CacheBF16 {
  static constexpr bool kFp4 = false;
  using elem_t = uint16_t;
  __device__ static elem_t store(float x, float) { return f32_to_bf16_rne(x); }
};
struct CacheFP8 {
  static constexpr bool kFp4 = false;
  using elem_t = uint8_t;
  __device__ static elem_t store(float x, float scale) { return f32_to_e4m3_rne_sat(__fdiv_rn(x, scale)); }
};
// FP4 rows are written by fp4_append_blocks, not element by element.
struct CacheFP4 {
  static constexpr bool kFp4 = true;
  using elem_t = uint8_t;
  __device__ static elem_t store(float, float) { return 0; }
};

constexpr int kMxBlock = 32;

// E2M1 code of a value already divided by its block scale: nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even mantissa, saturating at 6;
// the sign bit is kept, so values that round to zero keep their sign.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float a = fabsf(q);
  uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | ((__float_as_uint(q) >> 28) & 0x8u);
}

// Four consecutive elements of a dtype (one 8-byte load for bf16).
template <class T>
struct alignas(4 * sizeof(T)) Vec4 {
  T v[4];
};

// Quantises this sequence's new K (rotated) and V rows, eight lanes per
// 32-element block (four elements each): codes to the block's code area at
// (slot, head), the scale byte to its scale area.  Each lane rotates its
// elements with the Q path's fp32 operations, the block's largest magnitude
// comes from three lane exchanges (a maximum, so in any order), and each
// lane rounds its four values and stores their two code bytes.  One thread
// per block did the same arithmetic as one serial chain per block, which
// set the kernel's time (12.9 us on 128 sequences of 8 kv heads).
template <class A>
__device__ void fp4_append_blocks(const AppendArgs& p, const typename A::elem_t* x, const float* s_cos,
                                  const float* s_sin, uint8_t* kblock, uint8_t* vblock, int slot, bool vec) {
#pragma clang fp contract(off)
  constexpr int kLanes = 8;                // lanes per block (aligned groups of a wave)
  constexpr int kPer = kMxBlock / kLanes;  // elements per lane
  static_assert(kThreads % kLanes == 0, "groups of eight lanes");
  const int D = p.dims.head_dim;
  const int half = D / 2;
  const int Hq = p.dims.num_q_heads;
  const int Hkv = p.dims.num_kv_heads;
  const int BS = p.dims.block_size;
  const int nblk = D / kMxBlock;
  const bool il = p.flags & LGM_ROPE_INTERLEAVED;
  const CacheStrides cc = cache_strides(p.flags, BS, Hkv, D / 2);         // code bytes
  const CacheStrides cs = cache_strides(p.flags, BS, Hkv, D / kMxBlock);  // scale bytes
  const int64_t codes_bytes = cc.block;
  // Every lane of a group runs the same iterations (the bound is a multiple
  // of kLanes), so the exchanges below always find their partners active.
  for (int t = threadIdx.x; t < 2 * Hkv * nblk * kLanes; t += kThreads) {
    const int q = t / kLanes;
    const int sub = t - q * kLanes;
    const bool is_v = q >= Hkv * nblk;
    const int u = is_v ? q - Hkv * nblk : q;
    const int g = u / nblk;
    const int blk = u - g * nblk;
    const typename A::elem_t* row = x + (int64_t)(Hq + (is_v ? Hkv : 0) + g) * D;
    // The block's elements k0 .. k0 + 3 of this lane and, for split-half K,
    // their rotation partners D/2 away (a block lies within one half, since
    // D/2 is a multiple of 32).  Interleaved pairs lie inside the lane's
    // elements (k0 is a multiple of 4).
    const int i_first = blk * kMxBlock;
    const int lo_first = (is_v || il) ? i_first : (i_first < half ? i_first : i_first - half);
    const int k0 = kPer * sub;
    typename A::elem_t xs[kPer], xp[kPer];  // x[i0 + k0 + k] and x[i0 + D/2 + k0 + k], i0 = lo_first
    if (vec) {
      using AV = Vec4<typename A::elem_t>;
      const AV a4 = *reinterpret_cast<const AV*>(row + lo_first + k0);
#pragma unroll
      for (int k = 0; k < kPer; ++k) xs[k] = a4.v[k];
      if (!is_v && !il) {
        const AV b4 = *reinterpret_cast<const AV*>(row + lo_first + half + k0);
#pragma unroll
        for (int k = 0; k < kPer; ++k) xp[k] = b4.v[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        xs[k] = row[lo_first + k0 + k];
        if (!is_v && !il) xp[k] = row[lo_first + half + k0 + k];
      }
    }
    float y[kPer];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      float v;
      if (is_v) {
        v = A::load(&xs[k]);
      } else if (il) {
        // the Q path's operations for pair (2i, 2i+1), i = (i_first + k0 + k) / 2
        const int i = (i_first + k0 + k) >> 1;
        const float c = s_cos[i];
        const float sn = s_sin[i];
        const float x0 = A::load(&xs[k & ~1]);
        const float x1 = A::load(&xs[k | 1]);
        if ((k & 1) == 0) {
          const float a0 = x0 * c;
          const float b0 = x1 * sn;
          v = a0 - b0;
        } else {
          const float a1 = x1 * c;
          const float b1 = x0 * sn;
          v = a1 + b1;
        }
      } else {
        // the Q path's operations for pair (i0, i0 + D/2)
        const int i0 = lo_first + k0 + k;
        const float c = s_cos[i0];
        const float sn = s_sin[i0];
        const float x0 = A::load(&xs[k]);
        const float x1 = A::load(&xp[k]);
        if (i_first < half) {
          const float a0 = x0 * c;
          const float b0 = x1 * sn;
          v = a0 - b0;
        } else {
          const float a1 = x1 * c;
          const float b1 = x0 * sn;
          v = a1 + b1;
        }
      }
      y[k] = v;
      amax = fmaxf(amax, fabsf(v));
    }
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int X = amax > 0.f ? ilogbf(amax) - 2 : -127;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    // 2^-X as an fp32 bit pattern: X <= 125 for any finite amax (ilogbf <= 127),
    // so the biased exponent 127 - X lies in [2, 254], a normal float.
    const float mul = __uint_as_float((uint32_t)(127 - X) << 23);
    uint32_t w = 0u;  // codes of elements k0 .. k0 + 3: bytes k0 / 2 and k0 / 2 + 1, low nibble first
#pragma unroll
    for (int k = 0; k < kPer; ++k) w |= e2m1_code(y[k] * mul) << (4 * k);
    uint8_t* base = (is_v ? vblock : kblock);
    uint8_t* dst = base + (int64_t)slot * cc.tok + (int64_t)g * cc.head + blk * (kMxBlock / 2) + k0 / 2;
    if ((uintptr_t)dst % 2 == 0) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
    } else {
      dst[0] = (uint8_t)w;
      dst[1] = (uint8_t)(w >> 8);
    }
    if (sub == 0) base[codes_bytes + (int64_t)slot * cs.tok + (int64_t)g * cs.head + blk] = (uint8_t)(X + 127);
  }
}

template <class A, class C>
__global__ __launch_bounds__(kThreads) void rope_kv_append_kernel(AppendArgs p) {
#pragma clang fp contract(off)
  __shared__ float s_cos[kMaxHalf];
  __shared__ float s_sin[kMaxHalf];

  const int b = blockIdx.x;
  const int D = p.dims.head_dim;
  const int half = D / 2;
  const int Hq = p.dims.num_q_heads;
  const int Hkv = p.dims.num_kv_heads;
  const int BS = p.dims.block_size;
  const int MB = p.dims.max_blocks_per_seq;

  int ctx = p.context_lens[b];
  const int cap = MB * BS;
  ctx = ctx > cap ? cap : ctx;
  const bool active = ctx >= 1;
  const int pos = active ? ctx - 1 : 0;

  // The slot's table entry is read before the rotation factors are computed,
  // so its latency overlaps theirs.
  bool write = false;
  int pb = 0;
  const CacheStrides cs = cache_strides(p.flags, BS, Hkv, D);  // in elements
  int64_t slot_base = 0;  // element offset of (block, slot, head 0, 0); head g adds g * cs.head
  if (active) {
    pb = p.block_tables[(int64_t)b * MB + pos / BS];
    write = (unsigned)pb < (unsigned)p.dims.num_blocks;
    slot_base = (int64_t)pb * cs.block + (int64_t)(pos % BS) * cs.tok;
  }
  const bool il = p.flags & LGM_ROPE_INTERLEAVED;
  // Heads rotated by the element paths: Q and K, or only Q for FP4 caches,
  // whose K rows are rotated block by block in fp4_append_blocks.
  const int nrot_heads = Hq + (C::kFp4 ? 0 : Hkv);
  for (int i = threadIdx.x; i < half; i += kThreads) {
    const double w = pow((double)p.rope_theta, (-2.0 * (double)i) / (double)D);
    const double ang = (double)pos * w;
    double sd, cd;
    sincos(ang, &sd, &cd);
    s_cos[i] = (float)cd;
    s_sin[i] = (float)sd;
  }
  __syncthreads();

  const typename A::elem_t* x = static_cast<const typename A::elem_t*>(p.qkv) + (int64_t)b * p.qkv_row_stride;
  typename A::elem_t* qo = static_cast<typename A::elem_t*>(p.q_out) + (int64_t)b * Hq * D;
  typename C::elem_t* kc = static_cast<typename C::elem_t*>(p.k_cache);
  typename C::elem_t* vc = static_cast<typename C::elem_t*>(p.v_cache);

  // Eight-element vectors when every row and pointer allows them (the usual
  // case: dense packed QKV); element by element otherwise.  The arithmetic is
  // the same either way.
  const bool vec = (half % 8 == 0) && ((uintptr_t)p.qkv % (8 * sizeof(typename A::elem_t)) == 0) &&
                   ((p.qkv_row_stride * (int64_t)sizeof(typename A::elem_t)) % (8 * sizeof(typename A::elem_t)) == 0) &&
                   ((uintptr_t)p.q_out % (8 * sizeof(typename A::elem_t)) == 0) &&
                   ((uintptr_t)p.k_cache % (8 * sizeof(typename C::elem_t)) == 0) &&
                   ((uintptr_t)p.v_cache % (8 * sizeof(typename C::elem_t)) == 0);
  // Stores rotated head hh (Q, or K head hh - Hq) element e.
  auto store_rot = [&](int hh, int e, float y) {
    if (hh < Hq) {
      qo[hh * D + e] = A::store(y);
    } else if (write) {
      const int g = hh - Hq;
      kc[slot_base + (int64_t)g * cs.head + e] = C::store(y, p.k_scale ? kv_scale(p.k_scale, p.flags, g) : 1.f);
    }
  };
  if (vec) {
    using AV = Vec8<typename A::elem_t>;
    using CV = Vec8<typename C::elem_t>;
    const int nchunk = half / 8;
    // Rotate every Q head (and K head): nrot_heads * D/16 chunks of 8 pairs,
    // (i0 .. i0+7, i0+D/2 .. i0+D/2+7) split-half or (2i0 .. 2i0+15) interleaved.
    for (int t = threadIdx.x; t < nrot_heads * nchunk; t += kThreads) {
      const int hh = t / nchunk;
      const int i0 = 8 * (t - hh * nchunk);
      const int e_lo = il ? 2 * i0 : i0;          // first element of each 8-element vector
      const int e_hi = il ? 2 * i0 + 8 : i0 + half;
      const AV lo = *reinterpret_cast<const AV*>(x + hh * D + e_lo);
      const AV hi = *reinterpret_cast<const AV*>(x + hh * D + e_hi);
      float y0[8], y1[8];  // split-half: y[i0+k], y[i0+D/2+k]; interleaved: y[2i0+k], y[2i0+8+k]
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // pair k: split-half (lo[k], hi[k]); interleaved (e[2k], e[2k+1]) of lo|hi
        const int ic = i0 + k;
        const float c = s_cos[ic];
        const float sn = s_sin[ic];
        float x0, x1;
        if (il) {
          x0 = A::load(k < 4 ? &lo.v[2 * k] : &hi.v[2 * k - 8]);
          x1 = A::load(k < 4 ? &lo.v[2 * k + 1] : &hi.v[2 * k - 7]);
        } else {
          x0 = A::load(&lo.v[k]);
          x1 = A::load(&hi.v[k]);
        }
        const float a0 = x0 * c;
        const float b0 = x1 * sn;
        const float r0 = a0 - b0;
        const float a1 = x1 * c;
        const float b1 = x0 * sn;
        const float r1 = a1 + b1;
        if (il) {
          float* dst = k < 4 ? y0 : y1;
          dst[(2 * k) & 7] = r0;
          dst[(2 * k + 1) & 7] = r1;
        } else {
          y0[k] = r0;
          y1[k] = r1;
        }
      }
      if (hh < Hq) {
        AV o0, o1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          o0.v[k] = A::store(y0[k]);
          o1.v[k] = A::store(y1[k]);
        }
        *reinterpret_cast<AV*>(qo + hh * D + e_lo) = o0;
        *reinterpret_cast<AV*>(qo + hh * D + e_hi) = o1;
      } else if (write) {
        const int g = hh - Hq;
        const float sc = p.k_scale ? kv_scale(p.k_scale, p.flags, g) : 1.f;
        CV o0, o1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          o0.v[k] = C::store(y0[k], sc);
          o1.v[k] = C::store(y1[k], sc);
        }
        typename C::elem_t* kh = kc + slot_base + (int64_t)g * cs.head;
        *reinterpret_cast<CV*>(kh + e_lo) = o0;
        *reinterpret_cast<CV*>(kh + e_hi) = o1;
      }
    }
    // V heads are stored unrotated.
    if (write && !C::kFp4) {
      const typename A::elem_t* xv = x + (Hq + Hkv) * D;
      for (int t = threadIdx.x; t < Hkv * D / 8; t += kThreads) {
        const int g = (8 * t) / D;
        const float sc = p.v_scale ? kv_scale(p.v_scale, p.flags, g) : 1.f;
        const AV in = *reinterpret_cast<const AV*>(xv + 8 * t);
        CV o;
#pragma unroll
        for (int k = 0; k < 8; ++k) o.v[k] = C::store(A::load(&in.v[k]), sc);
        *reinterpret_cast<CV*>(vc + slot_base + (int64_t)g * cs.head + (8 * t - g * D)) = o;
      }
    }
  } else {
    // Rotate every Q head (and K head): nrot_heads * D/2 pairs.
    const int nrot = nrot_heads * half;
    for (int t = threadIdx.x; t < nrot; t += kThreads) {
      const int hh = t / half;
      const int i = t - hh * half;
      const float c = s_cos[i];
      const float s = s_sin[i];
      const int e0 = il ? 2 * i : i;          // the pair's elements
      const int e1 = il ? 2 * i + 1 : i + half;
      const float x0 = A::load(x + hh * D + e0);
      const float x1 = A::load(x + hh * D + e1);
      const float a0 = x0 * c;
      const float b0 = x1 * s;
      const float y0 = a0 - b0;
      const float a1 = x1 * c;
      const float b1 = x0 * s;
      const float y1 = a1 + b1;
      store_rot(hh, e0, y0);
      store_rot(hh, e1, y1);
    }
    // V heads are stored unrotated.
    if (write && !C::kFp4) {
      const typename A::elem_t* xv = x + (Hq + Hkv) * D;
      for (int t = threadIdx.x; t < Hkv * D; t += kThreads) {
        const int g = t / D;
        const float sc = p.v_scale ? kv_scale(p.v_scale, p.flags, g) : 1.f;
        vc[slot_base + (int64_t)g * cs.head + (t - g * D)] = C::store(A::load(xv + t), sc);
      }
    }
  }
  if constexpr (C::kFp4) {
    if (write) {
      const int64_t block_bytes = (int64_t)BS * Hkv * (D / 2 + D / kMxBlock);
      fp4_append_blocks<A>(p, x, s_cos, s_sin, static_cast<uint8_t*>(p.k_cache) + (int64_t)pb * block_bytes,
                           static_cast<uint8_t*>(p.v_cache) + (int64_t)pb * block_bytes, pos % BS, vec);
    }
  }
}


template <class A, class C>
hipError_t launch(const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rope_kv_append_kernel<A, C>), dim3(a.dims.num_seqs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_kv_append(const AppendArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s) {
  if (act == LGM_F32 && cache == LGM_F32) return launch<ActF32, CacheF32>(a, s);
  if (act == LGM_BF16 && cache == LGM_BF16) return launch<ActBF16, CacheBF16>(a, s);
  if (act == LGM_BF16 && cache == LGM_FP8_E4M3) return launch<ActBF16, CacheFP8>(a, s);
  if (act == LGM_BF16 && cache == LGM_FP4_E2M1) return launch<ActBF16, CacheFP4>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
