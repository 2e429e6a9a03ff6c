// Split-K paged GQA decode attention with matrix cores, for gfx950: bf16 or
// FP8 E4M3 caches, head_dim 128, block_size 16, group size G <= 16.
//
// The method is the one of paged_decode.hip (mainarch README, decode-attention
// section; Loom Kernels README, "Attention" row): partitions of the context
// processed by independent workgroups with an online softmax, merged by
// log-sum-exp, each KV row read once for its G query heads.  What changes is
// how a wave spends its instructions: with G query heads sharing a KV head,
// the scores of a 16-token block and the probability-weighted sum of V rows
// are small dense contractions, so both go to v_mfma_f32_16x16x32_bf16 and
// the vector ALU only runs the softmax bookkeeping.
//
// Operand layouts and the per-tile update are in mfma_common.h.  The
// probabilities enter the MFMA rounded to bf16 and the output is normalised by
// the sum of those same rounded values, so it is an exact convex combination
// of V rows up to fp32 accumulation; the log-sum-exp uses the unrounded sum.
#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

template <class C, int G>
__global__ __launch_bounds__(kDecodeThreads, 3) void paged_decode_mfma_kernel(DecodeArgs p) {
  static_assert(G >= 1 && G <= 16, "group size");
  __shared__ float s_acc[kNW][G][kD];
  __shared__ float s_m[kNW][G];
  __shared__ float s_l[kNW][G];   // sums of the bf16-rounded probabilities (normalise the output)
  __shared__ float s_le[kNW][G];  // sums of the fp32 probabilities (the log-sum-exp)

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = p.dims.num_q_heads;
  const int Hkv = p.dims.num_kv_heads;
  const int MB = p.dims.max_blocks_per_seq;
  const int PS = p.partition_size;

  int ctx = p.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  const int nparts = ctx == 0 ? 1 : (ctx + PS - 1) / PS;
  if (part >= nparts) return;
  const int start = part * PS;
  const int end = min(start + PS, ctx);

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int n = lane & 15;
  const int kg = lane >> 4;

  // Query rows as the B operand of the score MFMAs (bf16 bit patterns).
  short8 qb[4];
  {
    const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_seq_stride + (int64_t)g * G * kD;
    load_q_operand<C, G>(qb, qrow, qvec, n, kg);
  }
  float sscale = p.softmax_scale * kLog2e;
  if constexpr (C::kFp8) sscale *= p.k_scale[g];

  WaveState st;
  st.reset();

  const int32_t* bt = p.block_tables + (int64_t)b * MB;
  const int tok_bytes = Hkv * kD * C::kElemBytes;
  const int64_t block_bytes = (int64_t)kBS * tok_bytes;
  const int k_off = C::k_lane_off(g, tok_bytes, n, kg);
  const int v_off = C::v_lane_off(g, tok_bytes, n, kg);
  const unsigned nblocks = (unsigned)p.dims.num_blocks;
  const int lb_end = (end + kBS - 1) / kBS;

  const int lb0 = start / kBS;
  const int ntiles = (end - start + kTile - 1) / kTile;
  // Block ids of this wave's tiles, preloaded 32 tiles at a time into one
  // register (lane 2k + h holds block h of the wave's k-th tile) and read back
  // with readlane: no table load sits between a tile and its K/V loads.
  // -1 marks an absent block (past the end) or an out-of-range table entry.
  const __amdgpu_buffer_rsrc_t bt_rs = span_rsrc(bt, MB * 4);
  auto preload_ids = [&](int k0) -> int {
    const int t = wave + kNW * (k0 + (lane >> 1));
    const int lb = lb0 + 2 * t + (lane & 1);
    const int id = buf_load4(bt_rs, 4 * (lb < MB ? lb : 0));
    return (t < ntiles && lb < lb_end && (unsigned)id < nblocks) ? id : -1;
  };
  // Every tile issues the same loads: an absent or invalid block reads the
  // tile's other block (or block 0) instead and is masked, so the load count
  // per tile is fixed and the compiler can wait for K without waiting for V.
  auto tile_ids = [&](int ids, int k, int& px, int& py) {
    px = __builtin_amdgcn_readlane(ids, 2 * (k & 31));
    py = __builtin_amdgcn_readlane(ids, 2 * (k & 31) + 1);
  };

  // One register set per operand: the next tile's K loads are issued as soon
  // as the score MFMAs have consumed the current K, and its V loads as soon as
  // the output MFMAs have consumed the current V, so loads stay in flight
  // through all of a tile's arithmetic.
  TileRegs<C> tr;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kNW - 1) / kNW : 0;
  if (my_tiles > 0) {
    int ids = preload_ids(0);
    int px, py;
    tile_ids(ids, 0, px, py);
    int ex = px >= 0 ? px : 0, ey = py >= 0 ? py : ex;
    C::load_k(tr.kx, block_rsrc(p.k_cache, block_bytes, ex), k_off, tok_bytes);
    C::load_k(tr.ky, block_rsrc(p.k_cache, block_bytes, ey), k_off, tok_bytes);
    __builtin_amdgcn_sched_barrier(0);  // K before V, as inside the loop
    C::load_v(tr.vx, block_rsrc(p.v_cache, block_bytes, ex), v_off, tok_bytes);
    C::load_v(tr.vy, block_rsrc(p.v_cache, block_bytes, ey), v_off, tok_bytes);
    for (int k = 0; k < my_tiles; ++k) {
      const int t = wave + kNW * k;
      float4v sx, sy;
      tile_scores<C>(tr, qb, sx, sy);
      // Next tile's K.  After the last tile the current blocks are read again
      // (cache hits, results unused) so that every iteration issues the same
      // loads in the same order and the compiler can wait for K alone.
      const bool more = k + 1 < my_tiles;
      int nx = px, ny = py;
      if (more) {
        if (((k + 1) & 31) == 0) ids = preload_ids(k + 1);
        tile_ids(ids, k + 1, nx, ny);
        ex = nx >= 0 ? nx : 0;
        ey = ny >= 0 ? ny : ex;
      }
      C::load_k(tr.kx, block_rsrc(p.k_cache, block_bytes, ex), k_off, tok_bytes);
      C::load_k(tr.ky, block_rsrc(p.k_cache, block_bytes, ey), k_off, tok_bytes);
      tile_update<C>(st, tr, sx, sy, sscale, px >= 0, py >= 0, start + kTile * t, end, kg);
      C::load_v(tr.vx, block_rsrc(p.v_cache, block_bytes, ex), v_off, tok_bytes);
      C::load_v(tr.vy, block_rsrc(p.v_cache, block_bytes, ey), v_off, tok_bytes);
      px = nx;
      py = ny;
    }
  }

  // Wave epilogue: complete the denominators and publish this wave's state.
  const float lsum = sum4(st.lsum);
  const float lsum_e = sum4(st.lsum_e);
  if (kg == 0 && n < G) {
    s_m[wave][n] = st.m;
    s_l[wave][n] = lsum;
    s_le[wave][n] = lsum_e;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    if (h < G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_acc[wave][h][8 * n + i] = st.acc[i][j];
    }
  }
  __syncthreads();

  const float vscale = C::kFp8 ? p.v_scale[g] : 1.f;
  for (int idx = threadIdx.x; idx < G * kD; idx += kDecodeThreads) {
    const int h = idx / kD;
    const int d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w][h]);
    const float ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, Le = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = fast_exp2(s_m[w][h] - ms);
      L += s_l[w][h] * f;
      Le += s_le[w][h] * f;
      o += s_acc[w][h][d] * f;
    }
    o = L > 0.f ? o / L : 0.f;
    o *= vscale;
    const float lse = Le > 0.f ? (ms + fast_log2(Le)) * kLn2 : -INFINITY;
    const int64_t row = (int64_t)b * Hq + g * G + h;
    if (nparts == 1) {
      static_cast<uint16_t*>(p.out)[row * kD + d] = f32_to_bf16_rne(o);
      if (d == 0 && p.out_lse) p.out_lse[row] = lse;
    } else {
      p.part_out[(row * p.max_partitions + part) * kD + d] = o;
      if (d == 0) p.part_lse[row * p.max_partitions + part] = lse;
    }
  }
}

template <class C>
hipError_t dispatch(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid(a.max_partitions, a.dims.num_kv_heads, a.dims.num_seqs);
  const dim3 block(kDecodeThreads);
  switch (G) {
#define LGM_CASE(GV) \
  case GV: hipLaunchKernelGGL((paged_decode_mfma_kernel<C, GV>), grid, block, 0, s, a); break;
    LGM_CASE(1) LGM_CASE(2) LGM_CASE(3) LGM_CASE(4) LGM_CASE(5) LGM_CASE(6) LGM_CASE(7) LGM_CASE(8)
    LGM_CASE(9) LGM_CASE(10) LGM_CASE(11) LGM_CASE(12) LGM_CASE(13) LGM_CASE(14) LGM_CASE(15) LGM_CASE(16)
#undef LGM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size) {
  return act == LGM_BF16 && (cache == LGM_BF16 || cache == LGM_FP8_E4M3) && head_dim == kD && group >= 1 &&
         group <= 16 && block_size == kBS;
}

hipError_t launch_paged_decode_mfma(const DecodeArgs& a, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, G, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
