// Matrix-core building blocks shared by the decode kernels (gfx950,
// v_mfma_f32_16x16x32_bf16): cache formats, operand packing and the
// reductions over the four lanes that hold one head in the score layout.
//
// Operand mapping (lane l = 16*kg + n, kg = l / 16, n = l % 16):
//   scores  S^T[token][head] = K[token][d] * Q^T[d][head]: A = K rows (row n =
//           token n of a 16-token block; 8 consecutive head_dim values per
//           lane), B = the G query rows (column n = head n, zero for n >= G).
//           Output lane (kg, n) holds head n for tokens 4kg..4kg+3.
//   output  O[head][d] += P[head][token] * V[token][d]: A = the probabilities
//           exactly as the score MFMAs left them (row n = head n, 8 tokens per
//           lane: rows 4kg..4kg+3 of the two blocks of a 32-token tile); B = V
//           with column n of the i-th MFMA meaning head_dim index 8n + i, so a
//           lane needs V[token][8n .. 8n+7] of its 8 tokens: eight 16-byte
//           loads that together read whole 256-byte rows, and one byte
//           permute per operand register instead of a transpose.
//           Output lane (kg, n) holds O[head 4kg + j][8n + i] in acc[i][j].
// FP8 rows are converted to bf16 in registers (exact: every E4M3 value is a
// bf16 value).  FP4 rows (E2M1 codes, one E8M0 scale per 32 head-dim
// elements, stored after the block's codes) are converted to bf16 with their
// scale folded in by the scaled conversion (exact: an E2M1 value times a
// power of two has at most two significant bits).
#pragma once

#include "device_num.h"
#include "lgm_internal.h"

namespace lgm {
namespace mfma {

typedef short short8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kBS = 16;
constexpr int kTile = 32;  // tokens per wave iteration (two blocks)
constexpr int kNW = kDecodeThreads / kWaveSize;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ short8 words_to_short8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  uint4 u = make_uint4(w0, w1, w2, w3);
  return __builtin_bit_cast(short8, u);
}
// Two FP8 codes (low 16 bits of w) -> two bf16 packed in a dword (exact).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
// Reductions over the four lanes n, n+16, n+32, n+48 (one head in the score layout).
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- cache formats ------------------------------------------------------------
// Per 16-token block a lane holds: K for the score MFMAs (row n) and V for the
// output MFMAs (rows 4kg .. 4kg+3, head_dim 8n .. 8n+7).
// K/V reads go through buffer loads with one descriptor per 16-token block
// (base = the block, size = the block's bytes): offsets stay 32-bit for any
// pool size, a stray offset reads zeros instead of faulting, and the loads are
// intrinsic calls, which the compiler keeps where the software pipeline puts
// them (plain loads carried around the tile loop get merged into a single
// load at the loop head, right before their use).
// An absent block (pb < 0: past the segment, or an out-of-range table
// entry) gets a descriptor of size zero at the pool's start: every load
// through it returns zeros without touching memory, and the step masks it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* pool, int64_t block_bytes, int pb) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(pool) + (int64_t)max(pb, 0) * block_bytes), (short)0,
      pb >= 0 ? (int)block_bytes : 0, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ int buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Cache policies of K/V loads.  kStreamPolicy sets the non-temporal hint
// (bit nt): on MI355X a plain streaming read reaches ~7.1 TB/s with it
// against ~6.1 TB/s with the default policy (4 GiB read), and the whole-row
// kernel, which reads whole blocks once per call, gains as much.  The
// per-head partition kernel reads 256-byte slices of rows whose other slices
// other workgroups read later, and is faster with the default policy.  A hint
// only: the values read are the same.
constexpr int kDefaultPolicy = 0;
constexpr int kStreamPolicy = 2;
template <int POL>
__device__ __forceinline__ uint4 kv_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL));
}
template <int POL>
__device__ __forceinline__ uint2 kv_load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
}
// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane l's bytes land at lds + 16 l.  lds must be the same for the
// whole wave (it goes to M0).
template <int POL>
__device__ __forceinline__ void kv_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, POL);
}
template <int POL>
__device__ __forceinline__ uint32_t kv_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL);
}
template <int POL>
__device__ __forceinline__ uint32_t kv_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, POL);
}
// Device-scope accesses (cache-policy bit sc1) through a buffer descriptor,
// for records that one workgroup writes and another reads within a launch:
// each XCD has its own L2, which writes such stores through and does not
// serve such loads from a stale line, as the memory model's device-scope
// relaxed stores and loads do.
constexpr int kDeviceScope = 16;
__device__ __forceinline__ void store16_device(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r, off, 0,
                                         kDeviceScope);
}
__device__ __forceinline__ void store4_device(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ float4 load16_device(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
}
__device__ __forceinline__ float load4_device(__amdgpu_buffer_rsrc_t r, int off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kDeviceScope));
}

// E8M0 byte -> the fp32 scale 2^(b - 127): the byte is the fp32 exponent
// field, except 0 (2^-127, an fp32 subnormal) and 0xFF (NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : (b == 0xFFu ? 0x7FC00000u : b << 23));
}
// Byte strides of one pool for the loads below: K/V rows of kRowBytes per
// (token, kv head), NHD or HND (CacheStrides), and for FP4 the scale area
// that follows the block's codes, laid out the same way with 4 bytes a row.
struct KVLayout {
  int64_t block;  // bytes per block
  int tok;        // between consecutive tokens' rows of one head
  int head;       // between consecutive heads' rows of one token
  int sbase;      // FP4: first byte of the block's scale area
  int stok, shead;  // FP4: scale-row strides, as tok / head
};
template <class C>
__device__ __forceinline__ KVLayout kv_layout(uint32_t flags, int hkv) {
  const CacheStrides c = cache_strides(flags, kBS, hkv, C::kRowBytes);
  const CacheStrides sc = cache_strides(flags, kBS, hkv, C::kScaleRowBytes);
  return KVLayout{c.block + sc.block, c.tok, c.head, (int)c.block, sc.tok, sc.head};
}

// Two E2M1 codes (byte SEL of w, low nibble first) times scale -> two bf16 packed in a dword.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

struct MfmaBF16 {
  static constexpr bool kFp8 = false;
  static constexpr int kStepBlocks = 2;  // see step_blocks
  using elem_t = uint16_t;
  static constexpr int kRowBytes = kD * 2;  // one (token, kv head) row
  static constexpr int kScaleRowBytes = 0;
  __device__ static int score_d(int c, int kg, int j) { return 32 * c + 8 * kg + j; }
  struct KBlock {
    uint4 k[4];  // K[n][32c + 8kg .. +8], c = 0..3
  };
  struct VBlock {
    uint4 v[4];  // V[4kg + jj][8n .. +8], jj = 0..3
  };
  // Byte offsets inside a block of this lane's first K / V chunk (kv head g).
  __device__ static int k_lane_off(const KVLayout& L, int g, int n, int kg) { return n * L.tok + g * L.head + 16 * kg; }
  __device__ static int v_lane_off(const KVLayout& L, int g, int n, int kg) {
    return 4 * kg * L.tok + g * L.head + 16 * n;
  }
  __device__ static int k_scale_off(const KVLayout&, int, int, int) { return 0; }
  __device__ static int v_scale_off(const KVLayout&, int, int, int) { return 0; }
  template <int POL = kDefaultPolicy>
  __device__ static void load_k(KBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout&, int) {
#pragma unroll
    for (int c = 0; c < 4; ++c) r.k[c] = kv_load16<POL>(rs, off + 64 * c);
  }
  template <int POL = kDefaultPolicy>
  __device__ static void load_v(VBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout& L, int) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) r.v[jj] = kv_load16<POL>(rs, off + jj * L.tok);
  }
  // A operand of score MFMA c.
  __device__ static short8 k_operand(const KBlock& r, int c) { return __builtin_bit_cast(short8, r.k[c]); }
  // V elements i and i+1 (i even) of row jj, each packed with the same
  // element of row jj+1 -> two bf16x2 words (one byte permute each).
  __device__ static void v_pairs2(const VBlock& r, int jj, int i, uint32_t& lo, uint32_t& hi) {
    const uint32_t* a = reinterpret_cast<const uint32_t*>(&r.v[jj]);
    const uint32_t* b = reinterpret_cast<const uint32_t*>(&r.v[jj + 1]);
    const uint32_t x = a[i >> 1], y = b[i >> 1];
    lo = __builtin_amdgcn_perm(y, x, 0x05040100u);  // x.lo16 | y.lo16 << 16
    hi = __builtin_amdgcn_perm(y, x, 0x07060302u);  // x.hi16 | y.hi16 << 16
  }
  __device__ static void zero_v_row(VBlock& r, int jj) { r.v[jj] = make_uint4(0, 0, 0, 0); }
  __device__ static void prepare_v(VBlock&) {}
};

struct MfmaFP8 {
  static constexpr bool kFp8 = true;
  static constexpr int kStepBlocks = 2;
  using elem_t = uint8_t;
  static constexpr int kRowBytes = kD;
  static constexpr int kScaleRowBytes = 0;
  // Score MFMA c = 2u + h uses codes 8h .. 8h+7 of K chunk u.
  __device__ static int score_d(int c, int kg, int j) { return 64 * (c >> 1) + 16 * kg + 8 * (c & 1) + j; }
  struct KBlock {
    uint4 k[2];  // K[n][64u + 16kg .. +16] (16 codes), u = 0..1
  };
  struct VBlock {
    uint2 v[4];  // V[4kg + jj][8n .. +8] (8 codes)
  };
  __device__ static int k_lane_off(const KVLayout& L, int g, int n, int kg) { return n * L.tok + g * L.head + 16 * kg; }
  __device__ static int v_lane_off(const KVLayout& L, int g, int n, int kg) {
    return 4 * kg * L.tok + g * L.head + 8 * n;
  }
  __device__ static int k_scale_off(const KVLayout&, int, int, int) { return 0; }
  __device__ static int v_scale_off(const KVLayout&, int, int, int) { return 0; }
  template <int POL = kDefaultPolicy>
  __device__ static void load_k(KBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout&, int) {
#pragma unroll
    for (int u = 0; u < 2; ++u) r.k[u] = kv_load16<POL>(rs, off + 64 * u);
  }
  template <int POL = kDefaultPolicy>
  __device__ static void load_v(VBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout& L, int) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) r.v[jj] = kv_load8<POL>(rs, off + jj * L.tok);
  }
  // Score MFMA c = 2u + h uses codes 8h .. 8h+7 of K chunk u: head_dim 64u + 16kg + 8h + j.
  __device__ static short8 k_operand(const KBlock& r, int c) {
    const uint4& q = r.k[c >> 1];
    const uint32_t w0 = (c & 1) ? q.z : q.x;
    const uint32_t w1 = (c & 1) ? q.w : q.y;
    return words_to_short8(fp8x2_to_bf16x2(w0), fp8x2_hi_to_bf16x2(w0), fp8x2_to_bf16x2(w1),
                           fp8x2_hi_to_bf16x2(w1));
  }
  // Codes i and i+1 (i even) of rows jj and jj+1: one byte permute gathers
  // [row jj code i, row jj+1 code i, row jj code i+1, row jj+1 code i+1] and
  // the two halves convert to the two bf16x2 words.
  __device__ static void v_pairs2(const VBlock& r, int jj, int i, uint32_t& lo, uint32_t& hi) {
    const uint32_t x = i < 4 ? r.v[jj].x : r.v[jj].y;
    const uint32_t y = i < 4 ? r.v[jj + 1].x : r.v[jj + 1].y;
    const uint32_t q = __builtin_amdgcn_perm(y, x, (i & 3) == 0 ? 0x05010400u : 0x07030602u);
    lo = fp8x2_to_bf16x2(q);
    hi = fp8x2_hi_to_bf16x2(q);
  }
  __device__ static void zero_v_row(VBlock& r, int jj) { r.v[jj] = make_uint2(0, 0); }
  __device__ static void prepare_v(VBlock&) {}
};

// Lane x of a wave receives lane (x & ~3) + J's value (a quad broadcast).
template <int J>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, J * 0x55, 0xF, 0xF, false);
}

// FP4 blocks: codes [16][Hkv][64 bytes] (two E2M1 codes a byte, low nibble
// first), then scales [16][Hkv][4 bytes] (E8M0, one per 32 head-dim elements).
struct MfmaFP4 {
  static constexpr bool kFp8 = false;
  static constexpr int kStepBlocks = 2;
  using elem_t = uint8_t;
  static constexpr int kRowBytes = kD / 2;        // codes of one (token, kv head) row
  static constexpr int kScaleRowBytes = kD / 32;  // its scales
  // Lane kg holds head-dim 32kg .. 32kg+31 of its K row (one scale block);
  // score MFMA c takes eight of them.
  __device__ static int score_d(int c, int kg, int j) { return 32 * kg + 8 * c + j; }
  struct KBlock {
    uint4 k;     // codes of K[n][32kg .. 32kg+31]
    uint32_t s;  // their scale byte
  };
  // The V scales of a lane's four rows: lane (kg, 4a + t) loads the four
  // scale bytes of row 4kg + t, and the rows a lane reads (4kg .. 4kg + 3,
  // byte a) are then in its own quad: one dword load instead of four byte
  // loads, each of which costs the load pipeline a whole instruction.
  // prepare_v takes each row's byte from its quad neighbour once the loads
  // are in; a masked row keeps a finite scale (bit jj of dead).
  struct VBlock {
    uint32_t v[4];  // codes of V[4kg + jj][8n .. 8n+7]
    uint32_t sw;    // scale bytes of row 4kg + (n & 3)
    uint32_t dead;  // bit jj: row jj masked
    float sf[4];    // scales of rows 4kg + jj, head-dim block n / 4 (prepare_v)
  };
  __device__ static int k_lane_off(const KVLayout& L, int g, int n, int kg) { return n * L.tok + g * L.head + 16 * kg; }
  __device__ static int v_lane_off(const KVLayout& L, int g, int n, int kg) {
    return 4 * kg * L.tok + g * L.head + 4 * n;
  }
  // Scale bytes: the (token t, head g) row's four scales sit at
  // sbase + t * stok + g * shead; byte s covers head-dim 32s .. 32s+31.
  __device__ static int k_scale_off(const KVLayout& L, int g, int n, int kg) {
    return L.sbase + n * L.stok + g * L.shead + kg;
  }
  __device__ static int v_scale_off(const KVLayout& L, int g, int n, int kg) {
    return L.sbase + (4 * kg + (n & 3)) * L.stok + g * L.shead;
  }
  template <int POL = kDefaultPolicy>
  __device__ static void load_k(KBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout&, int soff) {
    r.k = kv_load16<POL>(rs, off);
    r.s = kv_load1<POL>(rs, soff);
  }
  template <int POL = kDefaultPolicy>
  __device__ static void load_v(VBlock& r, __amdgpu_buffer_rsrc_t rs, int off, const KVLayout& L, int soff) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) r.v[jj] = kv_load4<POL>(rs, off + jj * L.tok);
    r.sw = kv_load4<POL>(rs, soff);
    r.dead = 0;
  }
  // Every lane of a quad needs the same head-dim block (n / 4), so each lane
  // decodes its own row's scale for that block once and the quad shares the
  // decoded values.
  __device__ static void prepare_v(VBlock& r) {
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const uint32_t own = __float_as_uint(e8m0_to_f32((r.sw >> (8 * ((lane >> 2) & 3))) & 0xFFu));
    r.sf[0] = (r.dead & 1u) ? 1.f : __uint_as_float(quad_bcast<0>(own));
    r.sf[1] = (r.dead & 2u) ? 1.f : __uint_as_float(quad_bcast<1>(own));
    r.sf[2] = (r.dead & 4u) ? 1.f : __uint_as_float(quad_bcast<2>(own));
    r.sf[3] = (r.dead & 8u) ? 1.f : __uint_as_float(quad_bcast<3>(own));
  }
  __device__ static short8 k_operand(const KBlock& r, int c) {
    const uint32_t w = c == 0 ? r.k.x : (c == 1 ? r.k.y : (c == 2 ? r.k.z : r.k.w));
    const float sc = e8m0_to_f32(r.s);
    return words_to_short8(fp4x2_to_bf16x2<0>(w, sc), fp4x2_to_bf16x2<1>(w, sc), fp4x2_to_bf16x2<2>(w, sc),
                           fp4x2_to_bf16x2<3>(w, sc));
  }
  // Rows jj and jj+1, elements i and i+1 (i even, one byte of each row):
  // convert that byte of each row with the row's own scale, then pair the
  // halves.
  __device__ static void v_pairs2(const VBlock& r, int jj, int i, uint32_t& lo, uint32_t& hi) {
    uint32_t x, y;
    const float sx = r.sf[jj], sy = r.sf[jj + 1];
    switch (i >> 1) {
      case 0: x = fp4x2_to_bf16x2<0>(r.v[jj], sx); y = fp4x2_to_bf16x2<0>(r.v[jj + 1], sy); break;
      case 1: x = fp4x2_to_bf16x2<1>(r.v[jj], sx); y = fp4x2_to_bf16x2<1>(r.v[jj + 1], sy); break;
      case 2: x = fp4x2_to_bf16x2<2>(r.v[jj], sx); y = fp4x2_to_bf16x2<2>(r.v[jj + 1], sy); break;
      default: x = fp4x2_to_bf16x2<3>(r.v[jj], sx); y = fp4x2_to_bf16x2<3>(r.v[jj + 1], sy); break;
    }
    lo = __builtin_amdgcn_perm(y, x, 0x05040100u);  // element i of both rows
    hi = __builtin_amdgcn_perm(y, x, 0x07060302u);  // element i+1 of both rows
  }
  // A masked row: zero codes and (prepare_v) a finite scale, so the row
  // contributes exactly zero whatever its stored scale byte held.
  __device__ static void zero_v_row(VBlock& r, int jj) {
    r.v[jj] = 0;
    r.dead |= 1u << jj;
  }
};

// Head-dim index held by (MFMA c, lane group kg, slot j) in the score operands.
template <class C>
__device__ __forceinline__ int score_d(int c, int kg, int j) {
  return C::score_d(c, kg, j);
}

// Query rows of a head group as the B operand of the score MFMAs (bf16 bit
// patterns; zero for n >= G).  qrow points at head 0 of the group.  Aligned
// rows are read with 16-byte buffer loads (the same kind of load as the K/V
// stream, so the compiler can keep counting outstanding loads exactly);
// unaligned rows fall back to element loads.
template <class C, int G>
__device__ __forceinline__ void load_q_operand(short8 (&qb)[4], const uint16_t* qrow, bool vec, int n, int kg) {
  const int row = (n < G ? n : 0) * kD;  // rows n >= G read row 0 and are zeroed
  uint4 raw[4];
  if (vec) {
    const __amdgpu_buffer_rsrc_t rs = span_rsrc(qrow, G * kD * 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = buf_load16(rs, 2 * (row + score_d<C>(c, kg, 0)));
  } else {
    const uint16_t* qp = qrow + row;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)qp[score_d<C>(c, kg, 2 * j)] | ((uint32_t)qp[score_d<C>(c, kg, 2 * j + 1)] << 16);
      raw[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (n >= G) raw[c] = make_uint4(0, 0, 0, 0);
    qb[c] = __builtin_bit_cast(short8, raw[c]);
  }
}

// The score scale in log2 units (softmax_scale * log2(e), times the FP8 K
// scale), made positive so that max(scale * s) = scale * max(s): a negative
// scale flips the sign bits of the query operand instead, which is exact in
// bf16.  A zero scale becomes the smallest normal float, so that a masked
// score (-inf) still maps to -inf; every live score then maps to ~0, as it
// would with a zero scale.
__device__ __forceinline__ float fold_score_scale(float c, short8 (&qb)[4]) {
  if (c < 0.f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint4 u = __builtin_bit_cast(uint4, qb[k]);
      u.x ^= 0x80008000u;
      u.y ^= 0x80008000u;
      u.z ^= 0x80008000u;
      u.w ^= 0x80008000u;
      qb[k] = __builtin_bit_cast(short8, u);
    }
  }
  const float a = fabsf(c);
  return a == 0.f ? 1.17549435e-38f : a;
}

// Online-softmax state of one wave for one (sequence, kv head), against a
// lazily moved reference: m is the reference of head n in log2 units (the
// same in its four lanes; -inf until the head has a live score) and ms the
// offset the exponentials use (m, or 0 while m is -inf).  The reference moves
// only when a step's maximum passes it by more than kRescaleGap, so
// probabilities stay below 2^kRescaleGap and the accumulators are rescaled a
// handful of times per context instead of at every new maximum; any
// reference gives the same normalised output and log-sum-exp.
//   lsum_e  this lane's share of the sum of the fp32 probabilities (the LSE)
//   psum    sums of the bf16-rounded probabilities of heads 4kg .. 4kg+3
//           (from an MFMA against a column of ones; every column holds the
//           same sum): the output is normalised by the sum of the rounded
//           values it was built from, an exact convex combination of V rows
//   acc     acc[i][j] = O[head 4kg + j][8n + i]
constexpr float kRescaleGap = 8.f;

struct WaveState {
  float m, ms, lsum_e;
  float4v psum;
  float4v acc[8];
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    ms = 0.f;
    lsum_e = 0.f;
    psum = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
};

// Blocks of 16 tokens a wave takes per step (every format: 2, one 32-token
// tile).  The step code takes any even count.  Steps of 64 tokens for FP8
// (16 KB of K and V per step, the bytes of a bf16 step) halved the vector
// instructions per byte but made the FP8 call slower (136 against 127 us on
// 128 contexts of 1024..4096 tokens): a copy of the kernel that only loads
// reached 118.6 us with 32-token steps and 120.9 us with 64-token steps, so
// the FP8 call is bound by how the memory system serves the reads, not by
// the bytes each wave keeps in flight; the larger steps only added register
// pressure (SGPR spills).  FP4's eight-wave kernel spilled to scratch with
// 64-token steps.
template <class C>
constexpr int step_blocks() {
  return C::kStepBlocks;
}

// Registers of one step: NB consecutive 16-token blocks of one kv head.
template <class C, int NB>
struct StepRegs {
  typename C::KBlock k[NB];
  typename C::VBlock v[NB];
};

// Every step issues the same loads: an absent block's loads return zeros
// without touching memory (block_rsrc) and the step masks it, so the load
// count per step is fixed and the compiler can wait for K without waiting
// for V.
template <class C, int NB>
__device__ __forceinline__ void load_step_k(const DecodeArgs& p, int g, const int (&id)[NB], int lane,
                                            StepRegs<C, NB>& sr) {
  const KVLayout L = kv_layout<C>(p.flags, p.dims.num_kv_heads);
  const int off = C::k_lane_off(L, g, lane & 15, lane >> 4);
  const int soff = C::k_scale_off(L, g, lane & 15, lane >> 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) C::load_k(sr.k[b], block_rsrc(p.k_cache, L.block, id[b]), off, L, soff);
}
template <class C, int NB>
__device__ __forceinline__ void load_step_v(const DecodeArgs& p, int g, const int (&id)[NB], int lane,
                                            StepRegs<C, NB>& sr) {
  const KVLayout L = kv_layout<C>(p.flags, p.dims.num_kv_heads);
  const int off = C::v_lane_off(L, g, lane & 15, lane >> 4);
  const int soff = C::v_scale_off(L, g, lane & 15, lane >> 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) C::load_v(sr.v[b], block_rsrc(p.v_cache, L.block, id[b]), off, L, soff);
}

// Raw scores of a step: s[b][j] = <q_n, K[token 4kg + j of block b]>.
template <class C, int NB>
__device__ __forceinline__ void step_scores(const StepRegs<C, NB>& r, const short8 (&qb)[4], float4v (&s)[NB]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) s[b] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(C::k_operand(r.k[b], c), qb[c], s[b], 0, 0, 0);
  }
}

// Moves the reference of every head of the wave to max(m, ts) and rescales
// the sums and accumulators by 2^(m_old - m_new): row j of lane group kg is
// head 4kg + j, whose factor sits in lane 4kg + j.  Taken rarely; the
// rescaled accumulators go back through an MFMA with zero operands, so that
// outside this branch they stay in the registers the MFMAs use (a plain
// multiply made the compiler copy every accumulator out and back around the
// branch on every step).
__device__ __forceinline__ void rescale(WaveState& st, float ts, int kg) {
  const float mn = fmaxf(st.m, ts);
  const float ms = mn == -INFINITY ? 0.f : mn;
  const float alpha = fast_exp2(st.m - ms);  // 0 before the first live score
  st.m = mn;
  st.ms = ms;
  st.lsum_e *= alpha;
  float4v a4;
#pragma unroll
  for (int j = 0; j < 4; ++j) a4[j] = __shfl(alpha, 4 * kg + j);
  const short8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  st.psum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(z, z, st.psum * a4, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(z, z, st.acc[i] * a4, 0, 0, 0);
}

// Softmax update and output MFMAs of one step whose raw scores are s.
// csc: the positive score scale (fold_score_scale); valid: bit b set when
// block b is present with a valid table entry (uniform); tok0: first token
// of the step; end: one past the last valid token (same origin).  On an edge
// step (a block absent, or the context ending inside the step) masked rows
// get -inf scores and zeroed V rows: V there may hold anything, even NaN,
// and a zero probability must contribute exactly zero.
template <class C, int NB>
__device__ __forceinline__ void step_update(WaveState& st, StepRegs<C, NB>& r, float4v (&s)[NB], float csc,
                                            uint32_t valid, int tok0, int end, int kg) {
  static_assert(NB % 2 == 0, "steps are whole 32-token tiles");
  constexpr uint32_t kAll = (1u << NB) - 1u;
  if (__builtin_expect(valid != kAll || tok0 + NB * kBS > end, 0)) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!((valid >> b) & 1u) || tok0 + kBS * b + 4 * kg + j >= end) {
          s[b][j] = -INFINITY;
          C::zero_v_row(r.v[b], j);
        }
      }
    }
  }
  float tmax = s[0][0];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int j = (b == 0 ? 1 : 0); j < 4; ++j) tmax = fmaxf(tmax, s[b][j]);
  }
  tmax = max4(tmax);
  const float ts = tmax == -INFINITY ? -INFINITY : tmax * csc;
  if (__builtin_expect(__any(ts > st.m + kRescaleGap), 0)) rescale(st, ts, kg);
  // Probabilities 2^(csc * s - ms), rounded to bf16 once for the output
  // MFMAs.  P operand of block pair q: head n, tokens rows 4kg..4kg+3 of
  // block 2q then of block 2q+1, exactly as the score MFMAs left them.
  const float nms = -st.ms;
  const short8 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};  // bf16 1.0
  float pe = 0.f;
#pragma unroll
  for (int q = 0; q < NB / 2; ++q) {
    uint32_t pw[4];
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      const float4v& sb = s[2 * q + (t2 >> 1)];
      const float p0 = fast_exp2(fmaf(sb[2 * (t2 & 1)], csc, nms));
      const float p1 = fast_exp2(fmaf(sb[2 * (t2 & 1) + 1], csc, nms));
      pw[t2] = pack_bf16(p0, p1);
      pe += p0 + p1;
    }
    const short8 pa = words_to_short8(pw[0], pw[1], pw[2], pw[3]);
    st.psum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, st.psum, 0, 0, 0);
    C::prepare_v(r.v[2 * q]);  // (after the exponentials: the first use of this pair's V)
    C::prepare_v(r.v[2 * q + 1]);
    const typename C::VBlock& vx = r.v[2 * q];
    const typename C::VBlock& vy = r.v[2 * q + 1];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
      C::v_pairs2(vx, 0, i, a0, a1);
      C::v_pairs2(vx, 2, i, b0, b1);
      C::v_pairs2(vy, 0, i, c0, c1);
      C::v_pairs2(vy, 2, i, d0, d1);
      st.acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, words_to_short8(a0, b0, c0, d0), st.acc[i], 0, 0, 0);
      st.acc[i + 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, words_to_short8(a1, b1, c1, d1), st.acc[i + 1], 0, 0, 0);
    }
  }
  st.lsum_e += pe;
}

}  // namespace mfma
}  // namespace lgm
