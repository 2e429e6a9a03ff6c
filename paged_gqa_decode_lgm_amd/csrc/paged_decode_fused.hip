// Split-K paged decode attention in one launch, for jobs too small to fill
// the chip with whole contexts: gfx950 matrix cores, bf16 / FP8 / FP4 caches,
// head_dim 128, block_size 16, group size G <= 16.
//
// The method is the split-K decode of the other kernels (mainarch README,
// decode-attention section; Loom Kernels README, "Attention" row): each
// context is cut into partitions processed independently with an online
// softmax, and the partial results are combined by log-sum-exp.  On a small
// job the time is latency, not bandwidth: a second launch for the combine
// costs about as much as the attention itself.  So the combine runs in the
// same launch, in the workgroup that finishes a context's last partition.
//
// Grid: one workgroup per (sequence, kv head, partition); its four waves take
// the partition's 32-token steps in turn.  At entry the context length, the
// partition's block ids and the query are loaded together, and the first
// step's K/V loads follow as soon as the ids are back.  The four wave states
// are combined in LDS.  A context of one partition is written out directly.
// Otherwise the partition's normalised output and LSE (a record) are stored
// at device scope, and one lane counts the partition in with a device-scope
// atomic on the stream's arrival counter.  The workgroup that brings the
// count to the number of partitions sets the counter back to zero, reads
// every record of the stream at device scope and writes the combined output.
//
// Coherence across XCDs: each XCD has its own L2, and ordinary stores stay
// in it.  The records therefore use device-scope (sc1) stores and loads,
// which the L2 writes through and does not serve stale.  Each lane waits for
// its own record stores to complete (vmcnt 0) before the workgroup barrier
// that precedes the arrival atomic.  So every record a merging workgroup
// reads was complete, at device scope, before its partition was counted in.
#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

template <int G>
struct FusedSmem {
  float acc[kNW][G][kD];
  float m[kNW][G];
  float l[kNW][G];   // sums of the bf16-rounded probabilities (normalise the output)
  float le[kNW][G];  // sums of the fp32 probabilities (the log-sum-exp)
  float lse[kFusedMaxChunks * G];  // the merging workgroup's record LSEs, [partition][head]
  int last;
};

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}

// A wave's state into LDS: the reference and fp32 sum of head n from lane n,
// the rounded-probability sum of head 4kg + j from psum[j] of lane group kg,
// O[4kg + j][8n + i] from acc[i][j].
template <int G>
__device__ __forceinline__ void publish(FusedSmem<G>& sm, const WaveState& st, int lane, int wave) {
  const int n = lane & 15, kg = lane >> 4;
  const float lsum_e = sum4(st.lsum_e);
  if (kg == 0 && n < G) {
    sm.m[wave][n] = st.m;
    sm.le[wave][n] = lsum_e;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    if (h < G) {
      if (n == 0) sm.l[wave][h] = st.psum[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.acc[wave][h][8 * n + i] = st.acc[i][j];
    }
  }
}

template <class C, int G>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_fused_kernel(DecodeArgs p, FusedArgs f) {
  static_assert(G >= 1 && G <= 16, "group size");
  constexpr int NB = step_blocks<C>();
  constexpr int kStepTok = NB * kBS;
  constexpr int kItems = G * kD / 4;  // (head, 4 columns) items of one row group
  __shared__ FusedSmem<G> sm;
  const int lane = threadIdx.x % kWaveSize;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int Hkv = p.dims.num_kv_heads;
  const int u = blockIdx.x / f.nchunks;
  const int c = blockIdx.x - u * f.nchunks;
  const int b = u / Hkv;
  const int g = u - b * Hkv;
  const int chunk_tok = kNW * f.chunk_steps * kStepTok;
  const int start = c * chunk_tok;
  const int64_t row0 = (int64_t)b * p.dims.num_q_heads + (int64_t)g * G;  // output row of head 0

  // Context length, block ids and query: three independent loads.  Lane l
  // of a wave holds block l % NB of the wave's step l / NB (step t of the
  // partition = wave + 4 * (l / NB)).
  const int ctx_raw = p.context_lens[b];
  const int MB = p.dims.max_blocks_per_seq;
  const int lb = start / kBS + NB * (wave + kNW * (lane / NB)) + lane % NB;
  const __amdgpu_buffer_rsrc_t bt_rs = span_rsrc(p.block_tables + (int64_t)b * MB, MB * 4);
  const int id_raw = buf_load4(bt_rs, 4 * (lb < MB ? lb : 0));
  short8 qb[4];
  {
    const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_seq_stride + (int64_t)g * G * kD;
    load_q_operand<C, G>(qb, qrow, qvec, lane & 15, lane >> 4);
  }
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > p.max_context_len ? p.max_context_len : ctx_raw);
  if (start >= ctx) {  // uniform: the whole workgroup leaves before any barrier
    if (c == 0) {      // an empty context: out = 0, lse = -inf
      uint16_t* out = static_cast<uint16_t*>(p.out) + row0 * kD;
      for (int i = threadIdx.x; i < kItems; i += kDecodeThreads) store_bf16x4(out + 4 * i, 0.f, 0.f, 0.f, 0.f);
      if (p.out_lse && threadIdx.x < G) p.out_lse[row0 + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int end = min(ctx, start + chunk_tok);
  const int nch = (ctx + chunk_tok - 1) / chunk_tok;  // live partitions of this context
  const int lb_end = (end + kBS - 1) / kBS;
  const int ids = (lane < NB * f.chunk_steps && lb < lb_end && lb < MB &&
                   (unsigned)id_raw < (unsigned)p.dims.num_blocks)
                      ? id_raw
                      : -1;
  const int nsteps = (end - start + kStepTok - 1) / kStepTok;
  const int my_steps = nsteps > wave ? (nsteps - wave + kNW - 1) / kNW : 0;

  float cs = p.softmax_scale * kLog2e;
  if constexpr (C::kFp8) cs *= kv_scale(p.k_scale, p.flags, g);
  const float csc = fold_score_scale(cs, qb);

  WaveState st;
  st.reset();
  StepRegs<C, NB> sr;
  int pid[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) pid[bb] = my_steps > 0 ? __builtin_amdgcn_readlane(ids, bb) : -1;
  load_step_k<C, NB>(p, g, pid, lane, sr);
  __builtin_amdgcn_sched_barrier(0);  // K before V, as inside the step loop
  load_step_v<C, NB>(p, g, pid, lane, sr);
  for (int k = 0; k < my_steps; ++k) {
    float4v s[NB];
    step_scores<C, NB>(sr, qb, s);
    int nid[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) nid[bb] = k + 1 < my_steps ? __builtin_amdgcn_readlane(ids, NB * (k + 1) + bb) : -1;
    load_step_k<C, NB>(p, g, nid, lane, sr);
    uint32_t valid = 0;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) valid |= (pid[bb] >= 0 ? 1u : 0u) << bb;
    step_update<C, NB>(st, sr, s, csc, valid, start + kStepTok * (wave + kNW * k), end, lane >> 4);
    load_step_v<C, NB>(p, g, nid, lane, sr);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) pid[bb] = nid[bb];
  }
  publish<G>(sm, st, lane, wave);
  __syncthreads();

  // The partition's result: item i = (head i / 32, columns 4 (i % 32) ..).
  const float vscale = C::kFp8 ? kv_scale(p.v_scale, p.flags, g) : 1.f;
  const int64_t rec = (int64_t)u * f.nchunks + c;  // this partition's record
  const __amdgpu_buffer_rsrc_t ro_rs = span_rsrc(f.rec_out, f.rec_out_bytes);
  const __amdgpu_buffer_rsrc_t rl_rs = span_rsrc(f.rec_lse, f.rec_lse_bytes);
  for (int i = threadIdx.x; i < kItems; i += kDecodeThreads) {
    const int h = i / (kD / 4);
    const int d0 = 4 * (i % (kD / 4));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm.m[w][h]);
    const float ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, Le = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float fw = fast_exp2(sm.m[w][h] - ms);
      L += sm.l[w][h] * fw;
      Le += sm.le[w][h] * fw;
      const float4 a = *reinterpret_cast<const float4*>(&sm.acc[w][h][d0]);
      o[0] += a.x * fw;
      o[1] += a.y * fw;
      o[2] += a.z * fw;
      o[3] += a.w * fw;
    }
    const float inv = L > 0.f ? vscale / L : 0.f;
    const float lse = Le > 0.f ? (ms + fast_log2(Le)) * kLn2 : -INFINITY;
    if (nch == 1) {
      store_bf16x4(static_cast<uint16_t*>(p.out) + (row0 + h) * kD + d0, o[0] * inv, o[1] * inv, o[2] * inv,
                   o[3] * inv);
      if (d0 == 0 && p.out_lse) p.out_lse[row0 + h] = lse;
    } else {
      store16_device(ro_rs, (int)(((rec * G + h) * kD + d0) * 4),
                     make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv));
      if (d0 == 0) store4_device(rl_rs, (int)((rec * G + h) * 4), lse);
    }
  }
  if (nch == 1) return;

  // Count the partition in; the last one of the context merges.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    int* arrivals = f.arrivals + u;
    const int before = __hip_atomic_fetch_add(arrivals, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = before == nch - 1 ? 1 : 0;
    if (last) __hip_atomic_store(arrivals, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = last;
  }
  __syncthreads();
  if (!sm.last) return;

  // Merge: the LSEs of all partitions and the records of the first
  // kMergeBatch are requested together; later records follow in batches.
  constexpr int kMergeBatch = 8;
  constexpr int kPer = (kItems + kDecodeThreads - 1) / kDecodeThreads;  // items per thread: 1 or 2
  const int64_t rec0 = (int64_t)u * f.nchunks;
  float lv[(kFusedMaxChunks * G + kDecodeThreads - 1) / kDecodeThreads];
#pragma unroll
  for (int r = 0; r < (int)(sizeof(lv) / sizeof(lv[0])); ++r) {
    const int j = threadIdx.x + kDecodeThreads * r;
    lv[r] = j < nch * G ? load4_device(rl_rs, (int)((rec0 * G + j) * 4)) : -INFINITY;
  }
  float4 rv[kPer][kMergeBatch];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = threadIdx.x + kDecodeThreads * e;
    const int h = i / (kD / 4), d0 = 4 * (i % (kD / 4));
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      rv[e][k] = (i < kItems && k < nch) ? load16_device(ro_rs, (int)((((rec0 + k) * G + h) * kD + d0) * 4))
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int r = 0; r < (int)(sizeof(lv) / sizeof(lv[0])); ++r) {
    const int j = threadIdx.x + kDecodeThreads * r;
    if (j < nch * G) sm.lse[j] = lv[r];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = threadIdx.x + kDecodeThreads * e;
    if (i >= kItems) break;
    const int h = i / (kD / 4), d0 = 4 * (i % (kD / 4));
    float M = -INFINITY;
    for (int k = 0; k < nch; ++k) M = fmaxf(M, sm.lse[k * G + h]);
    const float ms = M == -INFINITY ? 0.f : M;
    float S = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    // A record of weight zero is left out by a select, so its bytes never
    // reach the sum.
    auto fold = [&](int k, const float4& v) {
      const float l = sm.lse[k * G + h];
      const float w = l == -INFINITY ? 0.f : expf(l - ms);
      S += w;
      a.x = w == 0.f ? a.x : fmaf(w, v.x, a.x);
      a.y = w == 0.f ? a.y : fmaf(w, v.y, a.y);
      a.z = w == 0.f ? a.z : fmaf(w, v.z, a.z);
      a.w = w == 0.f ? a.w : fmaf(w, v.w, a.w);
    };
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (k < nch) fold(k, rv[e][k]);
    for (int k0 = kMergeBatch; k0 < nch; k0 += kMergeBatch) {
      float4 v[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        v[k] = k0 + k < nch ? load16_device(ro_rs, (int)((((rec0 + k0 + k) * G + h) * kD + d0) * 4))
                            : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        if (k0 + k < nch) fold(k0 + k, v[k]);
    }
    const float inv = S > 0.f ? 1.f / S : 0.f;
    store_bf16x4(static_cast<uint16_t*>(p.out) + (row0 + h) * kD + d0, a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    if (d0 == 0 && p.out_lse) p.out_lse[row0 + h] = S > 0.f ? M + logf(S) : -INFINITY;
  }
}

template <class C, int G>
hipError_t launch(const DecodeArgs& a, const FusedArgs& f, hipStream_t s) {
  const int64_t grid = (int64_t)a.dims.num_seqs * a.dims.num_kv_heads * f.nchunks;
  hipLaunchKernelGGL((paged_decode_fused_kernel<C, G>), dim3((unsigned)grid), dim3(kDecodeThreads), 0, s, a, f);
  return hipGetLastError();
}

template <class C>
hipError_t dispatch(const DecodeArgs& a, const FusedArgs& f, int G, hipStream_t s) {
  switch (G) {
#define LGM_CASE(GV) \
  case GV:           \
    return launch<C, GV>(a, f, s);
    LGM_CASE(1) LGM_CASE(2) LGM_CASE(3) LGM_CASE(4) LGM_CASE(5) LGM_CASE(6) LGM_CASE(7) LGM_CASE(8)
    LGM_CASE(9) LGM_CASE(10) LGM_CASE(11) LGM_CASE(12) LGM_CASE(13) LGM_CASE(14) LGM_CASE(15) LGM_CASE(16)
#undef LGM_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_paged_decode_fused(const DecodeArgs& a, const FusedArgs& f, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (f.chunk_steps < 1 || f.chunk_steps > kWaveSize / step_blocks<MfmaBF16>() || f.nchunks < 1 ||
      f.nchunks > kFusedMaxChunks)
    return hipErrorInvalidValue;
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, f, G, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, f, G, s);
  if (cache == LGM_FP4_E2M1) return dispatch<MfmaFP4>(a, f, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
