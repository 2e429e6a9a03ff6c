// Balanced ("stream") paged GQA decode attention for gfx950: bf16 / FP8 E4M3
// caches, head_dim 128, block_size 16, G <= 16, one launch.
//
// The split-KV method of the pages (mainarch README, decode-attention
// section: the cache is split across workgroups, each keeps a running max and
// sum, the partial results are combined; Loom Kernels README, "Attention"
// row: local split-K with an LSE merge) with the split points chosen for
// balance instead of at fixed token counts.  All (sequence, kv head)
// segments, each ceil(ctx / 32) tiles of 32 tokens, are laid end to end; wave
// w of W' = min(W, N) takes the tiles [w*N/W', (w+1)*N/W') of that sequence
// and streams them
// with the double-pipelined K/V loads of the matrix-core tile step, so every
// wave reads the same number of KV bytes whatever the context lengths, and
// keeps its loads in flight from its first tile to its last.
//
// A segment that lies inside one wave's range is written out directly.  A
// segment cut by range boundaries leaves one record per piece (unnormalised
// output rows, running max, both probability sums) in the workspace; the wave
// that completes the last piece (an atomic arrival count per segment) merges
// the records by log-sum-exp and writes the output, then resets the count to
// zero.  Hence the workspace contract: zero-filled before first use, left
// zeroed by every completed call.
#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

// Wave holding global tile i: the largest w with floor(w*N/W) <= i.
__device__ __forceinline__ int wave_of(int64_t i, int64_t N, int W) {
  return (int)(((i + 1) * W - 1) / N);
}
__device__ __forceinline__ int64_t range_lo(int w, int64_t N, int W) { return (int64_t)w * N / W; }

// Values every lane holds identically, made visibly uniform for the compiler
// (so they live in scalar registers and branch without exec masks).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& p, int b) {
  const int c = p.context_lens[b];
  return c < 0 ? 0 : (c > p.max_context_len ? p.max_context_len : c);
}

// Writes the normalised rows and the log-sum-exp of (b, g) from a wave's
// state (m, lr, le already summed over the four lanes of each head).
template <class C, int G>
__device__ void write_final(const DecodeArgs& p, int b, int g, const WaveState& st, float lr, float le, int n,
                            int kg) {
  const int Hq = p.dims.num_q_heads;
  const float vscale = C::kFp8 ? p.v_scale[g] : 1.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    const float lr_h = __shfl(lr, h);
    if (h < G) {
      const float inv = lr_h > 0.f ? vscale / lr_h : 0.f;
      uint4 o;
      o.x = pack_bf16(st.acc[0][j] * inv, st.acc[1][j] * inv);
      o.y = pack_bf16(st.acc[2][j] * inv, st.acc[3][j] * inv);
      o.z = pack_bf16(st.acc[4][j] * inv, st.acc[5][j] * inv);
      o.w = pack_bf16(st.acc[6][j] * inv, st.acc[7][j] * inv);
      uint16_t* dst = static_cast<uint16_t*>(p.out) + ((int64_t)b * Hq + g * G + h) * kD + 8 * n;
      *reinterpret_cast<uint4*>(dst) = o;
    }
  }
  if (p.out_lse && kg == 0 && n < G)
    p.out_lse[(int64_t)b * Hq + g * G + n] = le > 0.f ? (st.m + fast_log2(le)) * kLn2 : -INFINITY;
}

template <class C, int G>
__global__ __launch_bounds__(kWaveSize) __attribute__((amdgpu_waves_per_eu(stream_waves_per_simd(C::kFp8, G)))) void paged_decode_stream_kernel(
    DecodeArgs p, StreamArgs x) {
  static_assert(G >= 1 && G <= 16, "group size");
  constexpr int kRows = (G + 3) / 4;            // lane groups holding real head rows
  constexpr int kAccFloats = 16 * kRows * 32;   // accumulator part of a record
  const int w = blockIdx.x;
  const int W = x.num_waves;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int B = p.dims.num_seqs;
  const int Hq = p.dims.num_q_heads;
  const int Hkv = p.dims.num_kv_heads;
  const int MB = p.dims.max_blocks_per_seq;

  // Sequences with no context: output 0, log-sum-exp -inf.
  for (int b = w; b < B; b += W) {
    if (clamp_ctx(p, b) != 0) continue;
    for (int i = lane; i < Hq * kD / 8; i += kWaveSize)
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + (int64_t)b * Hq * kD)[i] = make_uint4(0, 0, 0, 0);
    if (p.out_lse)
      for (int h = lane; h < Hq; h += kWaveSize) p.out_lse[(int64_t)b * Hq + h] = -INFINITY;
  }

  // N = Hkv * sum_b ceil(ctx_b / 32), and the segment holding this wave's first tile.
  int64_t N = 0;
  for (int b0 = 0; b0 < B; b0 += kWaveSize) {
    const int b = b0 + lane;
    const int T = b < B ? (clamp_ctx(p, b) + kTile - 1) / kTile : 0;
    int s = T;
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) s += __shfl_xor(s, o);
    N += (int64_t)Hkv * uni(s);
  }
  if (N == 0) return;
  // Ranges are cut for min(W, N) waves so that every participating wave owns
  // at least one tile: the arrival count of a split segment then equals the
  // number of waves between its first and its last tile.
  const int Wr = (int)(N < (int64_t)W ? N : (int64_t)W);
  if (w >= Wr) return;
  const int64_t lo = range_lo(w, N, Wr);
  const int64_t hi = range_lo(w + 1, N, Wr);

  int b = 0;
  int64_t cb = 0;  // first global tile of sequence b
  int Tb = 0;      // tiles per segment of sequence b
  for (int b0 = 0;; b0 += kWaveSize) {
    const int bb = b0 + lane;
    const int T = bb < B ? (clamp_ctx(p, bb) + kTile - 1) / kTile : 0;
    int incl = T;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int64_t end_b = cb + (int64_t)Hkv * incl;  // one past the last tile of sequence bb
    const unsigned long long hit = __ballot(bb < B && end_b > lo);
    if (hit) {
      const int L = uni(__builtin_ctzll(hit));
      b = b0 + L;
      Tb = uni(__builtin_amdgcn_readlane(T, L));
      cb += (int64_t)Hkv * (uni(__builtin_amdgcn_readlane(incl, L)) - Tb);
      break;
    }
    cb += (int64_t)Hkv * uni(__builtin_amdgcn_readlane(incl, kWaveSize - 1));
  }
  int g = uni((int)((lo - cb) / Tb));

  const int tok_bytes = Hkv * kD * C::kElemBytes;
  const int64_t block_bytes = (int64_t)kBS * tok_bytes;
  const unsigned nblocks = (unsigned)p.dims.num_blocks;
  const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
  float* const rec_base = x.records;

  int64_t pos = lo;
  while (pos < hi) {
    const int64_t seg0 = cb + (int64_t)g * Tb;
    const int t_begin = (int)(pos - seg0);
    const int t_end = (int)((hi < seg0 + Tb ? hi : seg0 + Tb) - seg0);
    const int ctx = uni(clamp_ctx(p, b));
    const int lb_end = (ctx + kBS - 1) / kBS;
    const int32_t* bt = p.block_tables + (int64_t)b * MB;
    const int k_off = C::k_lane_off(g, tok_bytes, n, kg);
    const int v_off = C::v_lane_off(g, tok_bytes, n, kg);

    short8 qb[4];
    load_q_operand<C, G>(qb, static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_seq_stride + (int64_t)g * G * kD,
                         qvec, n, kg);
    float sscale = p.softmax_scale * kLog2e;
    if constexpr (C::kFp8) sscale *= p.k_scale[g];

    // Block ids of tiles t_begin + k, 32 tiles per preload (lane 2k + h holds block h of tile k).
    // (buffer loads over the table row: the same kind of load as the K/V stream)
    const __amdgpu_buffer_rsrc_t bt_rs = span_rsrc(bt, MB * 4);
    auto preload_ids = [&](int k0) -> int {
      const int t = t_begin + k0 + (lane >> 1);
      const int lb = 2 * t + (lane & 1);
      const int id = buf_load4(bt_rs, 4 * (lb < MB ? lb : 0));
      return (t < t_end && lb < lb_end && (unsigned)id < nblocks) ? id : -1;
    };
    WaveState st;
    st.reset();
    TileRegs<C> tr;
    const int ntl = t_end - t_begin;
    int ids = preload_ids(0);
    int px = __builtin_amdgcn_readlane(ids, 0), py = __builtin_amdgcn_readlane(ids, 1);
    int ex = px >= 0 ? px : 0, ey = py >= 0 ? py : ex;
    C::load_k(tr.kx, block_rsrc(p.k_cache, block_bytes, ex), k_off, tok_bytes);
    C::load_k(tr.ky, block_rsrc(p.k_cache, block_bytes, ey), k_off, tok_bytes);
    __builtin_amdgcn_sched_barrier(0);  // K before V, as inside the loop
    C::load_v(tr.vx, block_rsrc(p.v_cache, block_bytes, ex), v_off, tok_bytes);
    C::load_v(tr.vy, block_rsrc(p.v_cache, block_bytes, ey), v_off, tok_bytes);
    for (int k = 0; k < ntl; ++k) {
      float4v sx, sy;
      tile_scores<C>(tr, qb, sx, sy);
      // Next tile's K (the current blocks again after the last tile, so that
      // every iteration issues the same loads and K can be waited for alone).
      const bool more = k + 1 < ntl;
      int nx = px, ny = py;
      if (more) {
        if (((k + 1) & 31) == 0) ids = preload_ids(k + 1);
        nx = __builtin_amdgcn_readlane(ids, 2 * ((k + 1) & 31));
        ny = __builtin_amdgcn_readlane(ids, 2 * ((k + 1) & 31) + 1);
        ex = nx >= 0 ? nx : 0;
        ey = ny >= 0 ? ny : ex;
      }
      C::load_k(tr.kx, block_rsrc(p.k_cache, block_bytes, ex), k_off, tok_bytes);
      C::load_k(tr.ky, block_rsrc(p.k_cache, block_bytes, ey), k_off, tok_bytes);
      tile_update<C>(st, tr, sx, sy, sscale, px >= 0, py >= 0, kTile * (t_begin + k), ctx, kg);
      C::load_v(tr.vx, block_rsrc(p.v_cache, block_bytes, ex), v_off, tok_bytes);
      C::load_v(tr.vy, block_rsrc(p.v_cache, block_bytes, ey), v_off, tok_bytes);
      px = nx;
      py = ny;
    }

    const float lr = sum4(st.lsum);
    const float le = sum4(st.lsum_e);
    if (t_begin == 0 && t_end == Tb) {
      write_final<C, G>(p, b, g, st, lr, le, n, kg);
    } else {
      // Record of this piece: slot 0 for the wave's first piece, 1 for its last.
      float* rec = rec_base + ((int64_t)w * 2 + (pos == lo ? 0 : 1)) * x.record_floats;
      if (kg < kRows) {
        float4* dst = reinterpret_cast<float4*>(rec + lane * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = make_float4(st.acc[i][0], st.acc[i][1], st.acc[i][2], st.acc[i][3]);
      }
      if (kg == 0) {
        rec[kAccFloats + n] = st.m;
        rec[kAccFloats + 16 + n] = lr;
        rec[kAccFloats + 32 + n] = le;
      }
      __threadfence();
      int32_t* counter = x.counters + (int64_t)b * Hkv + g;
      int old = 0;
      if (lane == 0) old = atomicAdd(counter, 1);
      old = __builtin_amdgcn_readlane(old, 0);
      const int wa = wave_of(seg0, N, Wr);
      const int wb = wave_of(seg0 + Tb - 1, N, Wr);
      if (old == wb - wa) {
        // Last piece in: merge every record of the segment by log-sum-exp.
        __threadfence();
        const int64_t lo_wa = range_lo(wa, N, Wr);
        auto rec_of = [&](int xw) -> const float* {
          const int slot = (xw == wa && lo_wa < seg0) ? 1 : 0;
          return rec_base + ((int64_t)xw * 2 + slot) * x.record_floats;
        };
        float M = -INFINITY;
        for (int xw = wa; xw <= wb; ++xw) M = fmaxf(M, rec_of(xw)[kAccFloats + n]);
        const float Ms = M == -INFINITY ? 0.f : M;
        WaveState mg;
        mg.reset();
        float mlr = 0.f, mle = 0.f;
        for (int xw = wa; xw <= wb; ++xw) {
          const float* r = rec_of(xw);
          const float f = fast_exp2(r[kAccFloats + n] - Ms);
          mlr += r[kAccFloats + 16 + n] * f;
          mle += r[kAccFloats + 32 + n] * f;
          float fr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) fr[j] = __shfl(f, 4 * kg + j);
          if (kg < kRows) {
            const float4* src = reinterpret_cast<const float4*>(r + lane * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float4 v = src[i];
              mg.acc[i][0] += v.x * fr[0];
              mg.acc[i][1] += v.y * fr[1];
              mg.acc[i][2] += v.z * fr[2];
              mg.acc[i][3] += v.w * fr[3];
            }
          }
        }
        mg.m = Ms;
        write_final<C, G>(p, b, g, mg, mlr, mle, n, kg);
        if (lane == 0) *counter = 0;
      }
    }

    // Next segment.
    pos = seg0 + t_end;
    if (pos >= hi) break;
    if (++g == Hkv) {
      g = 0;
      cb += (int64_t)Hkv * Tb;
      do {
        ++b;
        Tb = b < B ? uni((clamp_ctx(p, b) + kTile - 1) / kTile) : 1;
      } while (Tb == 0);
      if (b >= B) break;
    }
  }
}

template <class C>
hipError_t dispatch(const DecodeArgs& a, const StreamArgs& x, int G, hipStream_t s) {
  const dim3 grid(x.num_waves);
  const dim3 block(kWaveSize);
  switch (G) {
#define LGM_CASE(GV) \
  case GV: hipLaunchKernelGGL((paged_decode_stream_kernel<C, GV>), grid, block, 0, s, a, x); break;
    LGM_CASE(1) LGM_CASE(2) LGM_CASE(3) LGM_CASE(4) LGM_CASE(5) LGM_CASE(6) LGM_CASE(7) LGM_CASE(8)
    LGM_CASE(9) LGM_CASE(10) LGM_CASE(11) LGM_CASE(12) LGM_CASE(13) LGM_CASE(14) LGM_CASE(15) LGM_CASE(16)
#undef LGM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int stream_record_floats(int group) {
  const int rows = (group + 3) / 4;
  const int floats = 16 * rows * 32 + 48;
  return (floats + 63) / 64 * 64;
}

hipError_t launch_paged_decode_stream(const DecodeArgs& a, const StreamArgs& x, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, x, G, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, x, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
