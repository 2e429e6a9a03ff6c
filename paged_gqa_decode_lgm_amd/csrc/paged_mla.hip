// Paged multi-head latent attention (MLA) decode for gfx950 matrix cores
// (mainarch README, MLA section: a paged latent cache of FP8 E4M3 ckv (512
// per token) beside bf16 kpe (64), per-head dot scores, local softmax with
// exported LSE, softmax-weighted latent output tiles, split-K across the
// sequence with a stage-2 merge of the partial records).
//
// Every query head attends to the same latent rows, so one wave takes all
// heads (up to 16) of a sequence at once: they are the 16 columns of the
// score MFMA and the 16 rows of the output MFMA (v_mfma_f32_16x16x32_bf16,
// lane l = 16 kg + n).
//   scores  S^T[token][head] = K[token][576] Q^T: 16 MFMAs over the latent
//           (FP8 codes converted to bf16, exactly) and 2 over the positional
//           part, in two accumulators, so that s = scale * (s_ckv * <q_lat,
//           code> + <q_pe, kpe>); lane (kg, n) reads 16 latent codes per
//           64-byte chunk and 8 positional values per 32 of token n.
//   output  O[head][512] += P[head][token] V[token][512], V = the latent
//           codes: 32 MFMAs per 32-token tile, column n of MFMA i meaning
//           latent element 32n + i, so a lane reads 32 contiguous bytes of
//           each of its 8 token rows; s_ckv is applied at the end.
// The latent bytes are therefore read twice per tile in the two operand
// layouts (once from HBM, once from cache).
//
// Work split: one workgroup per (sequence, partition); its four waves take
// the partition's 32-token tiles in turn (wave w: tiles w, w + 4, ...), each
// with its own running max and sums, and combine through LDS at the end, so
// a partition of ps tokens leaves one record however small ps / 4 is.  The
// record (normalised fp32 output and natural-log LSE) goes to the partial
// buffers when the sequence has several partitions (lse_merge combines
// them), else the output is written directly.
#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

constexpr int kDL = 512;  // latent elements
constexpr int kDR = 64;   // positional elements
constexpr int kDQ = kDL + kDR;
constexpr int kMlaWaves = kDecodeThreads / kWaveSize;
constexpr int kMlaHeads = 16;
constexpr int kMergePad = 36;
constexpr float kRescaleSlack = 8.f;  // floats per 32-element slice in the merge buffer (bank spread)

struct MlaMerge {
  float acc[kMlaWaves][kMlaHeads][16][kMergePad];  // [wave][head][n][i]: O[head][32n + i]
};
constexpr int kQRow = kDQ + 8;  // padded query row (bank spread of the operand reads)
union MlaSmem {
  uint16_t q[kMlaHeads][kQRow];  // query rows (bf16 bits), rows past num_heads zero
  MlaMerge m;                    // used once every wave has left its tile loop
};

// One 16-token half tile of one lane: K operands of token n (latent bytes
// 64u + 16kg .. +16, u < 8; positional elements 32c + 8kg .. +8, c < 2) and
// V operands of tokens 4kg + jj (latent bytes 32n .. 32n + 31).
struct MlaHalf {
  uint4 ck[8];
  uint4 kp[2];
  uint4 v[4][2];
};

__device__ __forceinline__ void load_k_half(const MlaArgs& p, int pb, int off, int lane, MlaHalf& h) {
  const int bs = p.dims.block_size;
  const int n = lane & 15, kg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rc = block_rsrc(p.ckv, (int64_t)bs * kDL, pb);
  const __amdgpu_buffer_rsrc_t rp = block_rsrc(p.kpe, (int64_t)bs * kDR * 2, pb);
#pragma unroll
  for (int u = 0; u < 8; ++u) h.ck[u] = kv_load16<kStreamPolicy>(rc, (off + n) * kDL + 64 * u + 16 * kg);
#pragma unroll
  for (int c = 0; c < 2; ++c) h.kp[c] = kv_load16<kStreamPolicy>(rp, (off + n) * kDR * 2 + 64 * c + 16 * kg);
}
__device__ __forceinline__ void load_v_half(const MlaArgs& p, int pb, int off, int lane, MlaHalf& h) {
  const int bs = p.dims.block_size;
  const int n = lane & 15, kg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rc = block_rsrc(p.ckv, (int64_t)bs * kDL, pb);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    h.v[jj][0] = kv_load16<kDefaultPolicy>(rc, (off + 4 * kg + jj) * kDL + 32 * n);
    h.v[jj][1] = kv_load16<kDefaultPolicy>(rc, (off + 4 * kg + jj) * kDL + 32 * n + 16);
  }
}

// Latent score MFMA c (0..15): codes 8(c & 1) .. +7 of chunk c >> 1.
__device__ __forceinline__ short8 latent_operand(const MlaHalf& h, int c) {
  const uint4& q = h.ck[c >> 1];
  const uint32_t w0 = (c & 1) ? q.z : q.x;
  const uint32_t w1 = (c & 1) ? q.w : q.y;
  return words_to_short8(fp8x2_to_bf16x2(w0), fp8x2_hi_to_bf16x2(w0), fp8x2_to_bf16x2(w1), fp8x2_hi_to_bf16x2(w1));
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int w) {
  return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
}
// Codes i and i + 1 (i even) of rows jj and jj + 1, interleaved as
// (row jj: i, row jj+1: i, row jj: i+1, row jj+1: i+1) by one byte permute.
__device__ __forceinline__ uint32_t code_pairs(const MlaHalf& h, int jj, int i) {
  const int s = i >> 4, w = (i >> 2) & 3;
  const uint32_t sel = (i & 2) ? 0x07030602u : 0x05010400u;
  return __builtin_amdgcn_perm(word_of(h.v[jj + 1][s], w), word_of(h.v[jj][s], w), sel);
}

// Query operands come from LDS at each use: held in registers they would
// push the tile's loads out of the register file.
__device__ __forceinline__ void half_scores(const MlaHalf& h, const uint16_t* qrow, int kg, float4v& s_lat,
                                            float4v& s_pe) {
  s_lat = (float4v){0.f, 0.f, 0.f, 0.f};
  s_pe = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const short8 qb = *reinterpret_cast<const short8*>(qrow + 64 * (c >> 1) + 16 * kg + 8 * (c & 1));
    s_lat = __builtin_amdgcn_mfma_f32_16x16x32_bf16(latent_operand(h, c), qb, s_lat, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const short8 qb = *reinterpret_cast<const short8*>(qrow + kDL + 32 * c + 8 * kg);
    s_pe = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(short8, h.kp[c]), qb, s_pe, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kDecodeThreads, 1) void paged_mla_kernel(MlaArgs p) {
  __shared__ MlaSmem sm;
  __shared__ float s_m[kMlaWaves][kMlaHeads], s_l[kMlaWaves][kMlaHeads], s_le[kMlaWaves][kMlaHeads];
  const int b = blockIdx.y;
  const int part = blockIdx.x;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int H = p.dims.num_heads;
  const int bs = p.dims.block_size;
  int ctx = p.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  const int PS = p.partition_size;
  const int nparts = ctx == 0 ? 1 : (ctx + PS - 1) / PS;
  if (part >= nparts) return;  // whole workgroup, before any barrier

  const float s_ckv = p.ckv_scale ? p.ckv_scale[0] : 1.f;
  const float sl2 = p.softmax_scale * kLog2e;
  const int t0 = part * PS;
  const int t1 = min(ctx, t0 + PS);
  const int32_t* bt = p.block_tables + (int64_t)b * p.dims.max_blocks_per_seq;
  const unsigned nb = (unsigned)p.dims.num_blocks;
  // Block and in-block offset of the half tile starting at token t; block -1
  // when t is past the partition or the table entry is out of range (the
  // loads then read block 0 and the tokens are masked).
  auto half_at = [&](int t, int& pb, int& off) {
    off = t % bs;
    pb = -1;
    if (t < t1) {
      const int id = __builtin_amdgcn_readfirstlane(bt[t / bs]);
      pb = (unsigned)id < nb ? id : -1;
    }
  };
  constexpr int kStride = kMlaWaves * kTile;
  MlaHalf hx, hy;
  int px, ox, py, oy;
  const int tw = t0 + wave * kTile;
  half_at(tw, px, ox);
  half_at(tw + 16, py, oy);
  // The sequence's query rows (latent then positional) into LDS, loaded
  // ahead of the first tile's K/V loads (which overlap the staging).
  {
    constexpr int kChunks = kMlaHeads * kDQ / 8;
    constexpr int kPer = (kChunks + kDecodeThreads - 1) / kDecodeThreads;
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + (int64_t)b * H * kDL;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q_pe) + (int64_t)b * H * kDR;
    uint4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {  // unconditional loads (clamped rows), zeroed after
      const int i = min(threadIdx.x + k * kDecodeThreads, kChunks - 1);
      const int row = i / (kDQ / 8);
      const int col = 8 * (i - row * (kDQ / 8));
      const int r = min(row, H - 1);
      v[k] = col < kDL ? *reinterpret_cast<const uint4*>(ql + r * kDL + col)
                       : *reinterpret_cast<const uint4*>(qp + r * kDR + (col - kDL));
    }
    // The first tile's loads follow, unconditionally (a wave with no tile
    // reads block 0 and never uses it), so that storing the query rows waits
    // for the query loads alone.
    __builtin_amdgcn_sched_barrier(0);
    load_k_half(p, px < 0 ? 0 : px, px < 0 ? 0 : ox, lane, hx);
    load_k_half(p, py < 0 ? 0 : py, py < 0 ? 0 : oy, lane, hy);
    load_v_half(p, px < 0 ? 0 : px, px < 0 ? 0 : ox, lane, hx);
    load_v_half(p, py < 0 ? 0 : py, py < 0 ? 0 : oy, lane, hy);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * kDecodeThreads;
      const int row = i / (kDQ / 8);
      const int col = 8 * (i - row * (kDQ / 8));
      if (i < kChunks) *reinterpret_cast<uint4*>(&sm.q[row][col]) = row < H ? v[k] : make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();
  const int n = lane & 15, kg = lane >> 4;
  const uint16_t* qrow = &sm.q[n][0];

  float m = -INFINITY, lsum = 0.f, lsum_e = 0.f;
  float4v acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = (float4v){0.f, 0.f, 0.f, 0.f};

  for (int t = tw; t < t1; t += kStride) {
    float4v lx, ex, ly, ey;
    half_scores(hx, qrow, kg, lx, ex);
    half_scores(hy, qrow, kg, ly, ey);
    const bool xval = px >= 0, yval = py >= 0;
    int nx, nox, ny, noy;
    half_at(t + kStride, nx, nox);
    half_at(t + kStride + 16, ny, noy);
    const bool more = t + kStride < t1;
    if (more) {  // next tile's K operands while this tile finishes
      load_k_half(p, nx < 0 ? 0 : nx, nx < 0 ? 0 : nox, lane, hx);
      load_k_half(p, ny < 0 ? 0 : ny, ny < 0 ? 0 : noy, lane, hy);
    }
    float s[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = (xval && t + 4 * kg + j < t1) ? sl2 * fmaf(s_ckv, lx[j], ex[j]) : -INFINITY;
      s[4 + j] = (yval && t + 16 + 4 * kg + j < t1) ? sl2 * fmaf(s_ckv, ly[j], ey[j]) : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // masked rows may hold any bytes (NaN codes)
      if (s[j] == -INFINITY) hx.v[j][0] = hx.v[j][1] = make_uint4(0, 0, 0, 0);
      if (s[4 + j] == -INFINITY) hy.v[j][0] = hy.v[j][1] = make_uint4(0, 0, 0, 0);
    }
    // Running reference max, moved only when a score passes it by more than
    // kRescaleSlack (log2 units): probabilities stay <= 2^kRescaleSlack, and
    // the accumulators are rescaled only on such a jump (any reference gives
    // the same normalised result and LSE).
    float tmax = s[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, s[j]);
    tmax = max4(tmax);
    const float mn = tmax > m + kRescaleSlack ? tmax : m;
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    const bool rescale = m != -INFINITY && mn != m;
    m = mn;
    uint32_t pw[4];
    float psum = 0.f, psum_e = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = fast_exp2(s[2 * k] - ms);
      const float p1 = fast_exp2(s[2 * k + 1] - ms);
      pw[k] = pack_bf16(p0, p1);
      psum += bf16_lo(pw[k]) + bf16_hi(pw[k]);
      psum_e += p0 + p1;
    }
    lsum = lsum * alpha + psum;
    lsum_e = lsum_e * alpha + psum_e;
    if (__any(rescale)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * kg + j);
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i][j] *= aj;
      }
    }
    const short8 pa = words_to_short8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const uint32_t a0 = code_pairs(hx, 0, i), a1 = code_pairs(hx, 2, i);
      const uint32_t a2 = code_pairs(hy, 0, i), a3 = code_pairs(hy, 2, i);
      const short8 v0 = words_to_short8(fp8x2_to_bf16x2(a0), fp8x2_to_bf16x2(a1), fp8x2_to_bf16x2(a2),
                                        fp8x2_to_bf16x2(a3));
      const short8 v1 = words_to_short8(fp8x2_hi_to_bf16x2(a0), fp8x2_hi_to_bf16x2(a1), fp8x2_hi_to_bf16x2(a2),
                                        fp8x2_hi_to_bf16x2(a3));
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, v0, acc[i], 0, 0, 0);
      acc[i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, v1, acc[i + 1], 0, 0, 0);
    }
    if (more) {
      load_v_half(p, nx < 0 ? 0 : nx, nx < 0 ? 0 : nox, lane, hx);
      load_v_half(p, ny < 0 ? 0 : ny, ny < 0 ? 0 : noy, lane, hy);
    }
    px = nx;
    ox = nox;
    py = ny;
    oy = noy;
  }

  // Combine the four waves.  Head h's max and sums sit in lanes h, h + 16,
  // h + 32, h + 48 of the score layout (the same value after the reductions);
  // acc[i][j] holds O[head 4kg + j][32n + i].
  const float ls = sum4(lsum), le = sum4(lsum_e);
  if (lane < kMlaHeads) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = ls;
    s_le[wave][lane] = le;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kMlaWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float f = fast_exp2(s_m[wave][h] - (M == -INFINITY ? 0.f : M));
    if (h < H) {
      float* dst = &sm.m.acc[wave][h][n][0];
#pragma unroll
      for (int i = 0; i < 32; i += 4)
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(acc[i][j] * f, acc[i + 1][j] * f, acc[i + 2][j] * f, acc[i + 3][j] * f);
    }
  }
  __syncthreads();
  const bool whole = nparts == 1;
  for (int e = threadIdx.x; e < H * (kDL / 2); e += kDecodeThreads) {  // two elements each
    const int h = e / (kDL / 2);
    const int d = 2 * (e - h * (kDL / 2));
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kMlaWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, Le = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) {
      const float f = fast_exp2(s_m[w][h] - Ms);
      L = fmaf(s_l[w][h], f, L);
      Le = fmaf(s_le[w][h], f, Le);
      const float2 v = *reinterpret_cast<const float2*>(&sm.m.acc[w][h][d >> 5][d & 31]);
      o0 += v.x;
      o1 += v.y;
    }
    const float inv = L > 0.f ? s_ckv / L : 0.f;
    const int64_t orow = (int64_t)b * H + h;
    const float lse = Le > 0.f ? (M + fast_log2(Le)) * kLn2 : -INFINITY;
    if (whole) {
      uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * kDL + d;
      *reinterpret_cast<uint32_t*>(dst) = (uint32_t)f32_to_bf16_rne(o0 * inv) | ((uint32_t)f32_to_bf16_rne(o1 * inv) << 16);
      if (d == 0 && p.out_lse) p.out_lse[orow] = lse;
    } else {
      const int64_t prow = orow * p.max_partitions + part;
      *reinterpret_cast<float2*>(p.part_out + prow * kDL + d) = make_float2(o0 * inv, o1 * inv);
      if (d == 0) p.part_lse[prow] = lse;
    }
  }
}

}  // namespace

bool mla_supported(lgm_dtype ckv, int latent_dim, int rope_dim, int num_heads, int block_size) {
  return ckv == LGM_FP8_E4M3 && latent_dim == kDL && rope_dim == kDR && num_heads >= 1 && num_heads <= kMlaHeads &&
         block_size >= 16 && block_size % 16 == 0;
}

hipError_t launch_paged_mla(const MlaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(paged_mla_kernel, dim3(a.max_partitions, a.dims.num_seqs), dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lgm
