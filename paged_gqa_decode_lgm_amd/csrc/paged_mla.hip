// Paged multi-head latent attention (MLA) decode for gfx950 matrix cores
// (mainarch README, MLA section: a paged latent cache of FP8 E4M3 ckv (512
// per token) beside bf16 kpe (64), per-head dot scores, local softmax with
// exported LSE, softmax-weighted latent output tiles, split-K across the
// sequence with a stage-2 merge of the partial records).
//
// Every query head attends to the same latent rows.  One workgroup takes one
// (sequence, partition) and walks it in 64-token tiles held in LDS.  Its
// eight waves have two roles:
//   load waves (4..7) gather the tiles through the block table into three
//           register stages and store them into one of three LDS tile
//           buffers two tiles ahead of the compute waves (loads are issued
//           five tiles ahead), so that HBM reads overlap the matrix work;
//           invalid rows (past the partition, or behind an out-of-range table
//           entry) are stored as zeros and masked.
//   compute waves (0..3), v_mfma_f32_16x16x32_bf16, lane l = 16 kg + n:
//     scores  wave w scores tokens 16w .. 16w+15 for all heads (up to 16,
//             the MFMA columns): S^T[token][head] = K[token][576] Q^T, 16
//             MFMAs over the latent (FP8 codes converted to bf16, exactly)
//             and 2 over the positional part in separate accumulators, so
//             that s = scale * (s_ckv * <q_lat, code> + <q_pe, kpe>);
//     softmax the waves exchange their tile maxima through LDS, so every
//             wave holds the same running reference max, and write their
//             probabilities (bf16) into a shared [head][token] tile;
//     output  wave w owns latent columns 128w .. 128w+127: O[head][col] +=
//             P[head][token] V[token][col], V = the latent codes, 8 MFMAs
//             per 32 tokens with column n of MFMA i meaning latent
//             128w + 8n + i, so a lane reads 8 contiguous codes of each of
//             its 8 token rows; s_ckv is applied at the end.
// Each latent byte is read from HBM once and converted twice (once per
// operand layout).  Two barriers per tile order the roles: B1 (tile maxima
// written) and B2 (probabilities written; the load waves then refill the
// buffer the previous tile used).  A partition's record (normalised fp32
// output and natural-log LSE) goes to the partial buffers when its sequence
// has several partitions (lse_merge combines them), else the output is
// written directly.
#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

constexpr int kDL = 512;  // latent elements
constexpr int kDR = 64;   // positional elements
constexpr int kMlaThreads = 512;
constexpr int kComputeWaves = 4;
constexpr int kMlaHeads = 16;
constexpr int kT = 64;               // tokens per tile
constexpr int kBufs = 3;             // LDS tile buffers
constexpr int kRowC = kDL + 16;      // LDS bytes per latent row (padded: bank spread)
constexpr int kRowP = 2 * kDR + 16;  // LDS bytes per positional row
constexpr int kRowPr = 2 * kT + 16;  // LDS bytes per probability row
constexpr float kRescaleSlack = 8.f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct MlaTileBuf {
  alignas(16) uint8_t ckv[kT * kRowC];
  alignas(16) uint8_t kpe[kT * kRowP];
  alignas(16) int32_t valid[kT];
};
struct MlaSmem {
  MlaTileBuf tile[kBufs];
  alignas(16) uint8_t prob[kMlaHeads * kRowPr];  // bf16 P[head][token] of the current tile
  float red[kComputeWaves][kMlaHeads];           // per-wave tile maxima, then final sums
  float red2[kComputeWaves][kMlaHeads];
};

// A load wave's share of a tile (load wave v = 0..3), in whole cache lines
// per load: latent load k (0..7) covers rows 8k + 2v and 8k + 2v + 1 (lane
// l: row 8k + 2v + l/32, bytes 16 (l % 32) .. +16); positional load k
// (0..1) covers rows 32k + 8v .. +8 (lane l: row 32k + 8v + l/8, bytes
// 16 (l % 8)).
struct MlaStage {
  u32x4 c[8];
  u32x4 r[2];
  int ok;  // bit k: latent row k valid; bit 8 + k: positional row k valid
};
__device__ __forceinline__ int lat_row(int k, int v, int lane) { return 8 * k + 2 * v + (lane >> 5); }
__device__ __forceinline__ int pos_row(int k, int v, int lane) { return 32 * k + 8 * v + (lane >> 3); }

__device__ __forceinline__ u32x4 ld_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Table entry of row `lane` of the tile starting at token ts (one load per
// lane; the rows a lane gathers take theirs from the lane of that row).  The
// read is clamped to the partition's last token (t1 - 1), so it stays within
// the entries of the context; the value is first used one tile later.
__device__ __forceinline__ int load_entry(const int32_t* bt, int ts, int t1, int bs_log2, int lane) {
  return bt[min(ts + lane, t1 - 1) >> bs_log2];
}

// Loads of this lane's share of the tile starting at ts; a row past the
// partition end t1 or behind an out-of-range entry reads block 0, row 0.
__device__ __forceinline__ void stage_load(const MlaArgs& p, int ts, int t1, int bs_log2, int entry, int v, int lane,
                                           MlaStage& st) {
  const unsigned nb = (unsigned)p.dims.num_blocks;
  const uint8_t* ckv = static_cast<const uint8_t*>(p.ckv);
  const uint8_t* kpe = static_cast<const uint8_t*>(p.kpe);
  int e[10];  // every row's entry first: one LDS round trip for all ten
#pragma unroll
  for (int k = 0; k < 10; ++k) e[k] = __shfl(entry, k < 8 ? lat_row(k, v, lane) : pos_row(k - 8, v, lane));
  int ok = 0;
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int tok = ts + (k < 8 ? lat_row(k, v, lane) : pos_row(k - 8, v, lane));
    const bool good = tok < t1 && (unsigned)e[k] < nb;
    // an invalid row reads block 0, row 0 (one line for all of them) and is zeroed after its store
    const int64_t row = ((int64_t)(good ? e[k] : 0) << bs_log2) + (good ? tok & ((1 << bs_log2) - 1) : 0);
    if (k < 8)
      st.c[k] = ld_nt(ckv + row * kDL + 16 * (lane & 31));
    else
      st.r[k - 8] = ld_nt(kpe + row * (2 * kDR) + 16 * (lane & 7));
    ok |= (int)good << k;
  }
  st.ok = ok;
}

// The rows go to LDS as loaded; only when a row of this wave's share is
// invalid (the partition's last tile, or an out-of-range table entry) are
// those rows overwritten with zeros (later LDS stores of one wave land later).
__device__ __forceinline__ void stage_store(const MlaStage& st, MlaTileBuf& tb, int v, int lane) {
  constexpr int kAll = (1 << 10) - 1;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    *reinterpret_cast<u32x4*>(&tb.ckv[lat_row(k, v, lane) * kRowC + 16 * (lane & 31)]) = st.c[k];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    *reinterpret_cast<u32x4*>(&tb.kpe[pos_row(k, v, lane) * kRowP + 16 * (lane & 7)]) = st.r[k];
  if (__builtin_expect(__any(st.ok != kAll), 0)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (!((st.ok >> k) & 1)) *reinterpret_cast<u32x4*>(&tb.ckv[lat_row(k, v, lane) * kRowC + 16 * (lane & 31)]) = z;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (!((st.ok >> (8 + k)) & 1)) *reinterpret_cast<u32x4*>(&tb.kpe[pos_row(k, v, lane) * kRowP + 16 * (lane & 7)]) = z;
  }
  if ((lane & 31) == 0) {  // one lane per latent row writes its flag
#pragma unroll
    for (int k = 0; k < 8; ++k) tb.valid[lat_row(k, v, lane)] = (st.ok >> k) & 1;
  }
}

__device__ __forceinline__ short8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return words_to_short8(fp8x2_to_bf16x2(w0), fp8x2_hi_to_bf16x2(w0), fp8x2_to_bf16x2(w1), fp8x2_hi_to_bf16x2(w1));
}

// Load waves: tiles 0 and 1 in LDS before the first barrier, then after
// each tile's B2 the tile two ahead into the buffer the previous tile used
// (its readers finished before this tile's B1), and a new load five ahead.
// Tile k sits in register stage k % 3; the table entries of its rows (one
// per lane) are loaded one step before the tile.  Tile starts past the partition are
// clamped to its last token (their rows are invalid and read block 0, row
// 0), so every load is unconditional and the memory counters carried around
// the loop are exact.
__device__ __forceinline__ void load_role(const MlaArgs& p, MlaSmem& sm, const int32_t* bt, int t0, int t1, int ntiles,
                                          int bsl, int v, int lane) {
  auto tile_start = [&](int k) { return min(t0 + k * kT, t1 - 1); };
  MlaStage s0, s1, s2;
  int e0 = load_entry(bt, tile_start(0), t1, bsl, lane);
  int e1 = load_entry(bt, tile_start(1), t1, bsl, lane);
  int e2 = load_entry(bt, tile_start(2), t1, bsl, lane);
  stage_load(p, tile_start(0), t1, bsl, e0, v, lane, s0);
  e0 = load_entry(bt, tile_start(3), t1, bsl, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(p, tile_start(1), t1, bsl, e1, v, lane, s1);
  e1 = load_entry(bt, tile_start(4), t1, bsl, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(p, tile_start(2), t1, bsl, e2, v, lane, s2);
  e2 = load_entry(bt, tile_start(5), t1, bsl, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(s0, sm.tile[0], v, lane);
  stage_load(p, tile_start(3), t1, bsl, e0, v, lane, s0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(s1, sm.tile[1], v, lane);
  stage_load(p, tile_start(4), t1, bsl, e1, v, lane, s1);
  __syncthreads();  // tiles 0 and 1 in LDS

  // Step tau: stage st holds tile tau+2 and entry eu that of tile tau+5;
  // el (free) takes that of tile tau+6.
  auto step = [&](int tau, MlaStage& st, int& eu, int& el) {
    __syncthreads();  // B1
    __syncthreads();  // B2
    if (tau + 2 < ntiles) stage_store(st, sm.tile[(tau + 2) % kBufs], v, lane);  // a tile past the end is never read
    el = load_entry(bt, tile_start(tau + 6), t1, bsl, lane);
    __builtin_amdgcn_sched_barrier(0);  // entry load ahead of the tile loads (counter order)
    stage_load(p, tile_start(tau + 5), t1, bsl, eu, v, lane, st);
  };
  int tau = 0;
  for (; tau + 2 < ntiles; tau += 3) {
    step(tau, s2, e2, e0);
    step(tau + 1, s0, e0, e1);
    step(tau + 2, s1, e1, e2);
  }
  if (tau < ntiles) step(tau, s2, e2, e0);
  if (tau + 1 < ntiles) step(tau + 1, s0, e0, e1);
  __syncthreads();  // final sums
  __builtin_amdgcn_s_waitcnt(0);  // drain the prefetches past the end before leaving
}

__global__ __launch_bounds__(kMlaThreads, 1) void paged_mla_kernel(MlaArgs p) {
  __shared__ MlaSmem sm;
  const int b = blockIdx.y;
  const int part = blockIdx.x;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int n = lane & 15, kg = lane >> 4;
  const int H = p.dims.num_heads;
  const int bsl = __builtin_ctz(p.dims.block_size);  // block_size is a power of two
  int ctx = p.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  const int PS = p.partition_size;
  const int nparts = ctx == 0 ? 1 : (ctx + PS - 1) / PS;
  if (part >= nparts) return;  // whole workgroup, before any barrier
  const int t0 = part * PS;
  const int t1 = min(ctx, t0 + PS);
  const int ntiles = t1 > t0 ? (t1 - t0 + kT - 1) / kT : 0;
  if (ntiles == 0) {  // an empty context (its one partition): zeros, LSE -inf
    if (w < kComputeWaves) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 4 * kg + j;
        if (h < H) {
          const int64_t orow = (int64_t)b * H + h;
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow * kDL + 128 * w + 8 * n) =
              make_uint4(0, 0, 0, 0);
          if (w == 0 && n == 0 && p.out_lse) p.out_lse[orow] = -INFINITY;
        }
      }
    }
    return;
  }
  const int32_t* bt = p.block_tables + (int64_t)b * p.dims.max_blocks_per_seq;
  if (w >= kComputeWaves) {
    load_role(p, sm, bt, t0, t1, ntiles, bsl, w - kComputeWaves, lane);
    return;
  }

  // ---- compute waves ----
  const float s_ckv = p.ckv_scale ? p.ckv_scale[0] : 1.f;
  const float sl2 = p.softmax_scale * kLog2e;
  // Query operands of head n: latent MFMA c reads elements 64(c>>1) + 16kg
  // + 8(c&1) .. +8, positional MFMA c 32c + 8kg .. +8.  Columns n >= H repeat
  // the last head (finite values whose rows are never written out).
  short8 qb[18];
  {
    const int hq = min(n, H - 1);
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + ((int64_t)b * H + hq) * kDL;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q_pe) + ((int64_t)b * H + hq) * kDR;
#pragma unroll
    for (int c = 0; c < 16; ++c) qb[c] = *reinterpret_cast<const short8*>(ql + 64 * (c >> 1) + 16 * kg + 8 * (c & 1));
#pragma unroll
    for (int c = 0; c < 2; ++c) qb[16 + c] = *reinterpret_cast<const short8*>(qp + 32 * c + 8 * kg);
  }
  float m = -INFINITY, lsum = 0.f, lsum_e = 0.f;
  float4v acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = (float4v){0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // tiles 0 and 1 in LDS

  for (int tau = 0; tau < ntiles; ++tau) {
    const MlaTileBuf& tb = sm.tile[tau % kBufs];
    float4v sl = {0.f, 0.f, 0.f, 0.f}, se = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* krow = &tb.ckv[(16 * w + n) * kRowC + 16 * kg];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 k = *reinterpret_cast<const u32x4*>(krow + 64 * u);
        sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(k.x, k.y), qb[2 * u], sl, 0, 0, 0);
        sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(k.z, k.w), qb[2 * u + 1], sl, 0, 0, 0);
      }
      const uint8_t* prow = &tb.kpe[(16 * w + n) * kRowP + 16 * kg];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        se = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const short8*>(prow + 64 * c), qb[16 + c], se,
                                                     0, 0, 0);
    }
    const int4 ok = *reinterpret_cast<const int4*>(&tb.valid[16 * w + 4 * kg]);
    float s[4];
    s[0] = ok.x ? sl2 * fmaf(s_ckv, sl[0], se[0]) : -INFINITY;
    s[1] = ok.y ? sl2 * fmaf(s_ckv, sl[1], se[1]) : -INFINITY;
    s[2] = ok.z ? sl2 * fmaf(s_ckv, sl[2], se[2]) : -INFINITY;
    s[3] = ok.w ? sl2 * fmaf(s_ckv, sl[3], se[3]) : -INFINITY;
    const float wmax = max4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    if (kg == 0) sm.red[w][n] = wmax;
    __syncthreads();  // B1
    // Shared reference max (the same in every wave), moved only when a score
    // passes it by more than kRescaleSlack (log2 units): probabilities stay
    // <= 2^kRescaleSlack and the accumulators are rescaled only on a jump.
    const float tmax = fmaxf(fmaxf(sm.red[0][n], sm.red[1][n]), fmaxf(sm.red[2][n], sm.red[3][n]));
    const float mn = tmax > m + kRescaleSlack ? tmax : m;
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    const bool rescale = m != -INFINITY && mn != m;
    m = mn;
    const float p0 = fast_exp2(s[0] - ms), p1 = fast_exp2(s[1] - ms);
    const float p2 = fast_exp2(s[2] - ms), p3 = fast_exp2(s[3] - ms);
    const uint32_t pw0 = pack_bf16(p0, p1), pw1 = pack_bf16(p2, p3);
    *reinterpret_cast<uint2*>(&sm.prob[n * kRowPr + (16 * w + 4 * kg) * 2]) = make_uint2(pw0, pw1);
    lsum = lsum * alpha + ((bf16_lo(pw0) + bf16_hi(pw0)) + (bf16_lo(pw1) + bf16_hi(pw1)));
    lsum_e = lsum_e * alpha + ((p0 + p1) + (p2 + p3));
    if (__any(rescale)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * kg + j);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][j] *= aj;
      }
    }
    __syncthreads();  // B2
#pragma unroll
    for (int s32 = 0; s32 < 2; ++s32) {  // two 32-token steps
      const short8 pa = *reinterpret_cast<const short8*>(&sm.prob[n * kRowPr + (32 * s32 + 8 * kg) * 2]);
      uint2 vr[8];  // codes 128w + 8n .. +8 of rows 32 s32 + 8kg + e
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vr[e] = *reinterpret_cast<const uint2*>(&tb.ckv[(32 * s32 + 8 * kg + e) * kRowC + 128 * w + 8 * n]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          // codes i = 4h + 2 i2 and i + 1 of rows (2 e2, 2 e2 + 1), interleaved
          const uint32_t sel = i2 ? 0x07030602u : 0x05010400u;
          uint32_t q[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            q[e2] = __builtin_amdgcn_perm(h ? vr[2 * e2 + 1].y : vr[2 * e2 + 1].x, h ? vr[2 * e2].y : vr[2 * e2].x, sel);
          const int i = 4 * h + 2 * i2;
          const short8 b0 = words_to_short8(fp8x2_to_bf16x2(q[0]), fp8x2_to_bf16x2(q[1]), fp8x2_to_bf16x2(q[2]),
                                            fp8x2_to_bf16x2(q[3]));
          const short8 b1 = words_to_short8(fp8x2_hi_to_bf16x2(q[0]), fp8x2_hi_to_bf16x2(q[1]),
                                            fp8x2_hi_to_bf16x2(q[2]), fp8x2_hi_to_bf16x2(q[3]));
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b0, acc[i], 0, 0, 0);
          acc[i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b1, acc[i + 1], 0, 0, 0);
        }
      }
    }
  }

  // Final sums over the compute waves (each summed its own tokens; all share m).
  const float ls = sum4(lsum), le = sum4(lsum_e);
  if (kg == 0) {
    sm.red[w][n] = ls;
    sm.red2[w][n] = le;
  }
  __syncthreads();  // final sums (the load waves join it)
  const bool whole = nparts == 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    const float L = (sm.red[0][h] + sm.red[1][h]) + (sm.red[2][h] + sm.red[3][h]);
    const float Le = (sm.red2[0][h] + sm.red2[1][h]) + (sm.red2[2][h] + sm.red2[3][h]);
    const float mh = __shfl(m, h);
    if (h < H) {
      const float inv = L > 0.f ? s_ckv / L : 0.f;
      const int64_t orow = (int64_t)b * H + h;
      const int col = 128 * w + 8 * n;
      const float lse = Le > 0.f ? (mh + fast_log2(Le)) * kLn2 : -INFINITY;
      if (whole) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (uint32_t)f32_to_bf16_rne(acc[2 * e][j] * inv) |
                 ((uint32_t)f32_to_bf16_rne(acc[2 * e + 1][j] * inv) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow * kDL + col) = make_uint4(o[0], o[1], o[2], o[3]);
        if (w == 0 && n == 0 && p.out_lse) p.out_lse[orow] = lse;
      } else {
        const int64_t prow = orow * p.max_partitions + part;
        float* dst = p.part_out + prow * kDL + col;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][j] * inv, acc[1][j] * inv, acc[2][j] * inv, acc[3][j] * inv);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(acc[4][j] * inv, acc[5][j] * inv, acc[6][j] * inv, acc[7][j] * inv);
        if (w == 0 && n == 0) p.part_lse[prow] = lse;
      }
    }
  }
}

}  // namespace

bool mla_supported(lgm_dtype ckv, int latent_dim, int rope_dim, int num_heads, int block_size) {
  return ckv == LGM_FP8_E4M3 && latent_dim == kDL && rope_dim == kDR && num_heads >= 1 && num_heads <= kMlaHeads &&
         block_size >= 1 && (block_size & (block_size - 1)) == 0;
}

hipError_t launch_paged_mla(const MlaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(paged_mla_kernel, dim3(a.max_partitions, a.dims.num_seqs), dim3(kMlaThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lgm
