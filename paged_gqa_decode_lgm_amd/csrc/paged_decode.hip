// Split-K paged GQA/MQA decode attention, vector-ALU form, for gfx950.
//
// The method (mainarch README, decode-attention section; Loom Kernels README,
// "Supported operator paths", row "Attention"): one query token per
// sequence attends over its paged KV cache; the context is cut into
// partitions processed by independent workgroups, each keeping an online
// softmax (running max and sum); GQA reads each KV head once for the G query
// heads sharing it; partial results are merged by log-sum-exp.
//
// Work decomposition.  Grid = (partition, kv head, sequence); one workgroup
// of 4 wave64s owns the G query heads of one kv head over one partition, so
// the K/V rows it streams are read once and used by all G heads from
// registers.  Waves take the partition's 16-token blocks round robin and
// double-buffer them (the next block's loads are in flight while the current
// one is processed).  Inside a wave, LPT = D / VEC lanes cover one token row
// with one 16-byte (8-byte for FP8) load each, so one load instruction reads
// TPI = 64 / LPT whole rows; each group of LPT lanes ("slot") keeps its own
// online-softmax state, and slots, then waves, are merged at the end.
// Scores are kept in log2 units (q is pre-scaled by softmax_scale * log2 e)
// so every exponential is a single v_exp_f32.
#include "device_num.h"
#include "lgm_internal.h"

namespace lgm {
namespace {

constexpr int kBS = 16;
constexpr int kNW = kDecodeThreads / kWaveSize;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// --- cache element formats: VEC elements of one token row per lane ------------
struct CacheF32 {
  using raw_t = float4;
  static constexpr int VEC = 4;
  static constexpr bool kFp8 = false;
  using elem_t = float;
  __device__ static void to_f32(const raw_t& r, float (&f)[VEC]) {
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
};
struct CacheBF16 {
  using raw_t = uint4;
  static constexpr int VEC = 8;
  static constexpr bool kFp8 = false;
  using elem_t = uint16_t;
  __device__ static void to_f32(const raw_t& r, float (&f)[VEC]) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};
struct CacheFP8 {
  using raw_t = uint2;
  static constexpr int VEC = 8;
  static constexpr bool kFp8 = true;
  using elem_t = uint8_t;
  __device__ static void to_f32(const raw_t& r, float (&f)[VEC]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = e4m3_to_f32((r.x >> (8 * i)) & 0xffu);
      f[4 + i] = e4m3_to_f32((r.y >> (8 * i)) & 0xffu);
    }
  }
};

// --- activation (q / out) formats -----------------------------------------------
struct ActF32 {
  using elem_t = float;
  __device__ static float load(const elem_t* p) { return *p; }
  __device__ static elem_t from_f32(float x) { return x; }
};
struct ActBF16 {
  using elem_t = uint16_t;
  __device__ static float load(const elem_t* p) { return bf16_to_f32(*p); }
  __device__ static elem_t from_f32(float x) { return f32_to_bf16_rne(x); }
};

template <class C, int U>
struct BlockRegs {
  typename C::raw_t k[U];
  typename C::raw_t v[U];
  bool ok[U];
};

template <class C, class A, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_split_kernel(DecodeArgs p) {
  constexpr int VEC = C::VEC;
  constexpr int LPT = D / VEC;          // lanes per token row
  constexpr int TPI = kWaveSize / LPT;  // token rows per load instruction
  constexpr int U = kBS / TPI;          // rows per lane per block
  static_assert(LPT >= 4 && LPT <= 32 && U >= 1 && kBS % TPI == 0, "unsupported lane mapping");
  using raw_t = typename C::raw_t;

  __shared__ float s_acc[kNW][G][D];
  __shared__ float s_m[kNW][G];
  __shared__ float s_l[kNW][G];

  // Partition index slowest: workgroups are dealt to the 8 XCDs by linear id,
  // and with the partition fastest an XCD would own fixed partition indices,
  // of which the high ones exist only for the longest sequences.
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int part = blockIdx.z;
  const int Hq = p.dims.num_q_heads;
  const int Hkv = p.dims.num_kv_heads;
  const int MB = p.dims.max_blocks_per_seq;

  int ctx = p.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  const int nparts = p.parts.count(ctx);
  if (part >= nparts) return;
  int start, end;
  p.parts.range(ctx, part, start, end);

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int slot = lane / LPT;
  const int chunk = lane % LPT;

  // q rows of the group, pre-scaled to log2 units (FP8: K's scale folded in).
  float qscale = p.softmax_scale * kLog2e;
  if constexpr (C::kFp8) qscale *= kv_scale(p.k_scale, p.flags, g);
  float q[G][VEC];
  {
    const typename A::elem_t* qp = static_cast<const typename A::elem_t*>(p.q) +
                                   (int64_t)b * p.q_seq_stride + (int64_t)g * G * D + chunk * VEC;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[h][e] = A::load(qp + h * D + e) * qscale;
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }

  const int32_t* bt = p.block_tables + (int64_t)b * MB;
  const typename C::elem_t* kc = static_cast<const typename C::elem_t*>(p.k_cache);
  const typename C::elem_t* vc = static_cast<const typename C::elem_t*>(p.v_cache);
  const CacheStrides cs = cache_strides(p.flags, kBS, Hkv, D);  // in elements
  const int64_t lane_off = (int64_t)g * cs.head + chunk * VEC;
  const unsigned nblocks = (unsigned)p.dims.num_blocks;

  auto load_block = [&](int lb, BlockRegs<C, U>& r) {
    const int pb = bt[lb];
    const bool blk_ok = (unsigned)pb < nblocks;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tib = u * TPI + slot;
      const int t = lb * kBS + tib;
      r.ok[u] = blk_ok && t < end;
      const int64_t off = (int64_t)pb * cs.block + (int64_t)tib * cs.tok + lane_off;
      raw_t zk{}, zv{};
      if (r.ok[u]) {
        zk = *reinterpret_cast<const raw_t*>(kc + off);
        zv = *reinterpret_cast<const raw_t*>(vc + off);
      }
      r.k[u] = zk;
      r.v[u] = zv;
    }
  };

  auto process_block = [&](const BlockRegs<C, U>& r) {
    float s[U][G];
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      C::to_f32(r.k[u], kf);
      C::to_f32(r.v[u], vf[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(q[h][e], kf[e], d);
        d = group_sum<LPT>(d);
        s[u][h] = r.ok[u] ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][h]);
      const float mn = fmaxf(m[h], mb);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - ms);
      float pu[U];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = fast_exp2(s[u][h] - ms);
        psum += pu[u];
      }
      l[h] = l[h] * alpha + psum;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a = acc[h][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(pu[u], vf[u][e], a);
        acc[h][e] = a;
      }
      m[h] = mn;
    }
  };

  const int lb_begin = start / kBS;
  const int lb_end = (end + kBS - 1) / kBS;
  BlockRegs<C, U> ra, rb;
  int lb = lb_begin + wave;
  if (lb < lb_end) load_block(lb, ra);
  for (; lb < lb_end; lb += 2 * kNW) {
    const int lb2 = lb + kNW;
    if (lb2 < lb_end) load_block(lb2, rb);
    process_block(ra);
    const int lb3 = lb2 + kNW;
    if (lb3 < lb_end) load_block(lb3, ra);
    if (lb2 < lb_end) process_block(rb);
  }

  // Merge the TPI slots of this wave (butterfly over the slot bits of the lane id).
#pragma unroll
  for (int off = LPT; off < kWaveSize; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float fa = fast_exp2(m[h] - ms);
      const float fb = fast_exp2(mo - ms);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = acc[h][e] * fa + __shfl_xor(acc[h][e], off) * fb;
      m[h] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_acc[wave][h][chunk * VEC + e] = acc[h][e];
      if (chunk == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves and write either the final row or this partition's record.
  const float vscale = C::kFp8 ? kv_scale(p.v_scale, p.flags, g) : 1.f;
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w][h]);
    const float ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = fast_exp2(s_m[w][h] - ms);
      L += s_l[w][h] * f;
      o += s_acc[w][h][d] * f;
    }
    o = L > 0.f ? o / L : 0.f;
    o *= vscale;
    const float lse = L > 0.f ? (ms + fast_log2(L)) * kLn2 : -INFINITY;
    const int64_t row = (int64_t)b * Hq + g * G + h;
    if (nparts == 1) {
      static_cast<typename A::elem_t*>(p.out)[row * D + d] = A::from_f32(o);
      if (d == 0 && p.out_lse) p.out_lse[row] = lse;
    } else {
      p.part_out[(row * p.max_partitions + part) * D + d] = o;
      if (d == 0) p.part_lse[row * p.max_partitions + part] = lse;
    }
  }
}

template <class C, class A, int D>
hipError_t dispatch_group(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid(a.dims.num_kv_heads, a.dims.num_seqs, a.max_partitions);
  const dim3 block(kDecodeThreads);
#define LGM_CASE(GV)                                                                    \
  case GV:                                                                              \
    hipLaunchKernelGGL((paged_decode_split_kernel<C, A, D, GV>), grid, block, 0, s, a); \
    break;
  switch (G) {
    LGM_CASE(1)
    LGM_CASE(2)
    LGM_CASE(3)
    LGM_CASE(4)
    LGM_CASE(5)
    LGM_CASE(6)
    LGM_CASE(7)
    LGM_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef LGM_CASE
  return hipGetLastError();
}

template <class C, class A>
hipError_t dispatch_dim(const DecodeArgs& a, int G, hipStream_t s) {
  if (a.dims.head_dim == 64) return dispatch_group<C, A, 64>(a, G, s);
  if (a.dims.head_dim == 128) return dispatch_group<C, A, 128>(a, G, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_valu_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size) {
  const bool types = (act == LGM_F32 && cache == LGM_F32) || (act == LGM_BF16 && cache == LGM_BF16) ||
                     (act == LGM_BF16 && cache == LGM_FP8_E4M3);
  return types && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8 && block_size == kBS;
}

bool decode_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size) {
  return decode_mfma_supported(act, cache, head_dim, group, block_size) ||
         decode_valu_supported(act, cache, head_dim, group, block_size);
}

// bf16 activations with bf16 / FP8 caches at head_dim 128 run on the matrix
// cores; every other supported shape runs the vector-ALU kernel above.
hipError_t launch_paged_decode(const DecodeArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (decode_mfma_supported(act, cache, a.dims.head_dim, G, a.dims.block_size))
    return launch_paged_decode_mfma(a, cache, s);
  if (act == LGM_F32 && cache == LGM_F32) return dispatch_dim<CacheF32, ActF32>(a, G, s);
  if (act == LGM_BF16 && cache == LGM_BF16) return dispatch_dim<CacheBF16, ActBF16>(a, G, s);
  if (act == LGM_BF16 && cache == LGM_FP8_E4M3) return dispatch_dim<CacheFP8, ActBF16>(a, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
