// Paged GQA decode attention over whole KV token rows, for gfx950 matrix
// cores: bf16 activations, bf16, FP8 E4M3 or FP4 E2M1 (E8M0 block scales)
// caches, head_dim 128, block_size 16, any kv head count.
//
// The split-K method of paged_decode.hip (mainarch README, decode-attention
// section; Loom Kernels README, "Attention" row) with the work laid out for
// how HBM serves a paged NHD cache.  A token row holds all kv heads side by
// side (Hkv x 256 bytes for bf16), and a 16-token block is one contiguous
// run of rows.  Workgroups that each read one kv head's 256-byte slice of
// every row leave the rest of each DRAM page to other workgroups at other
// times; here one workgroup covers a group of HG = 8 (or 4) kv heads, its four
// waves taking 2 (or 1) heads each, so the workgroup reads whole rows and
// whole blocks.  With 2 or 1 kv heads in all (or a count that 4 does not
// divide) the group is 2 or 1 heads and each head's steps are dealt to 2 or
// 4 waves in interleaved token slices (steps slice, slice + SL, ...), whose
// partial results the workgroup combines by log-sum-exp when it writes them:
// the workgroup still reads whole rows and the wave's pipeline is the same.
//
// The work is the flattened list of 32-token tiles of all streams (a stream
// is one sequence's tiles for one head group), cut into as many equal ranges
// as workgroups run at once: every workgroup reads the same number of bytes
// whatever the mix of context lengths, and there is no queue.  A range covers
// the end of one stream, whole streams, and the start of another; a stream
// that lies inside one range is written directly, the pieces of a split
// stream go to two record slots per workgroup and are merged by log-sum-exp
// afterwards (rows_merge_kernel).  Since each wave owns its heads (and token
// slice) for the whole range, no wave ever waits for another.
//
// Per tile a wave computes scores S^T = K Q^T and O += P V on
// v_mfma_f32_16x16x32_bf16 exactly as the partition kernel does (operand
// layouts and the softmax update in mfma_common.h), alternating between its
// two heads with one tile of loads in flight.
#include <type_traits>

#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

constexpr int kChunk = 1024;       // sequences per scan step
constexpr int kMaxRowWaves = 8;    // waves of the widest row workgroup
constexpr int kWin = 32;           // tiles per window of block ids (two ids per tile: one per lane)
constexpr int kStageWin = 4;       // windows of block ids staged in LDS per segment (128 tiles)

// A segment: the tiles lt .. et - 1 of one stream (sequence b, head group
// hg) that a range holds, and where its result goes.
struct SegDesc {
  int b, ctx, lt, et, hg, rec, whole, pad;
};

// Segments are processed in batches staged in LDS: their descriptors, the
// first window of their block ids, their query rows and (FP8) their kv-head
// scales, all loaded by the workgroup together, so that moving from one
// segment to the next costs no memory round trip; and their results, which
// the workgroup writes out together after the batch's last step.  (Results
// stored to global memory as each segment ended held up the loads issued
// after them, which wait for those stores to complete: 4-5 us per segment
// on 128 FP8 contexts of 1024..4096 tokens, measured with per-workgroup
// timestamps.)  A batch holds as many segments as ~108 KB of LDS allow; the
// FP8 kernel's K staging (32 KB, below) takes part of the rest.
template <int G, int HG, int SL>
struct Batch {
  static constexpr int kQRow = kD + 8;  // bf16 per staged query row; the pad spreads rows over LDS banks
  static constexpr int kPerSeg =
      HG * G * kQRow * 2 + SL * HG * G * (kD * 4 + 12) + kStageWin * 2 * kWin * 4 + 2 * HG * 4 + 32;
  static constexpr int kFit = 108000 / kPerSeg;
  static constexpr int kMax = kFit > 16 ? 16 : (kFit < 1 ? 1 : kFit);
};

template <int G, int HG, int SL>
struct RowsSmem {
  using B = Batch<G, HG, SL>;
  int pre[kChunk + 1];  // tiles of the streams of sequences b0 .. b0 + j - 1
  int wave_sum[kMaxRowWaves];
  SegDesc seg[B::kMax];
  int ids[B::kMax][kStageWin][2 * kWin];  // block ids of the segment's tiles lt .. lt + 127 (-1: absent)
  float kscale[B::kMax][HG];
  float vscale[B::kMax][HG];
  uint16_t q[B::kMax][HG * G][B::kQRow];
  // Results, row = (token slice * HG + local kv head) * G + query head of
  // the group: the accumulators and, per row, the rounded-probability sum
  // (psum), the fp32 sum (le) and the reference (ms) they are relative to;
  // the flush combines a head's slices and normalises them.
  float out[B::kMax][SL * HG * G][kD];
  float psum[B::kMax][SL * HG * G];
  float le[B::kMax][SL * HG * G];
  float ms[B::kMax][SL * HG * G];
};

__device__ __forceinline__ int clamped_ctx(const DecodeArgs& p, int b) {
  const int c = p.context_lens[b];
  return c < 0 ? 0 : (c > p.max_context_len ? p.max_context_len : c);
}

// Fills sm.pre for sequences b0 .. b0 + kChunk - 1 (nhg streams of
// ceil(ctx / unit) work units per sequence: 32-token tiles, or partitions;
// an empty context still counts one; each stream costs ucost per unit plus
// scost) and returns the chunk's total cost.  Called by every thread of the
// NT-thread workgroup (it synchronises).
template <int NT, class SM>
__device__ int scan_chunk(const DecodeArgs& p, SM& sm, int b0, int nhg, int unit, int min_units, int ucost,
                          int scost) {
  constexpr int SPT = kChunk / NT;  // sequences per thread
  static_assert(SPT * NT == kChunk && NT / kWaveSize <= kMaxRowWaves, "scan layout");
  const int tid = threadIdx.x, lane = tid & (kWaveSize - 1), wave = tid / kWaveSize;
  int t[SPT], s = 0;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int b = b0 + SPT * tid + k;
    t[k] = b < p.dims.num_seqs ? (max((clamped_ctx(p, b) + unit - 1) / unit, min_units) * ucost + scost) * nhg : 0;
    s += t[k];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) {
    const int x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  __syncthreads();  // earlier readers of sm.pre are done
  if (lane == kWaveSize - 1) sm.wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - s;
  for (int w = 0; w < wave; ++w) run += sm.wave_sum[w];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    sm.pre[SPT * tid + k] = run;
    run += t[k];
  }
  if (tid == NT - 1) sm.pre[kChunk] = run;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(sm.pre[kChunk]);
}

// Block ids of tiles k0 .. k0 + 31 of a segment starting at tile lt of
// sequence b, one per lane (lane 2k + h: block h of tile k0 + k); -1 marks a
// block past the segment or the context (lb_end blocks) or an out-of-range
// table entry.
__device__ __forceinline__ int preload_row_ids(const DecodeArgs& p, int b, int lt, int et, int lb_end, int k0,
                                               int lane) {
  const int MB = p.dims.max_blocks_per_seq;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc(p.block_tables + (int64_t)b * MB, MB * 4);
  const int tile = lt + k0 + (lane >> 1);
  const int lb = 2 * tile + (lane & 1);
  const int id = buf_load4(rs, 4 * (lb < MB ? lb : 0));
  return (tile < et && lb < lb_end && (unsigned)id < (unsigned)p.dims.num_blocks) ? id : -1;
}

// K/V load cache policy.  bf16 and FP8 head rows are whole 128-byte lines
// (or pairs of them) that one wave reads once, and the non-temporal hint lifts
// them to the streaming ceiling.  An FP4 head row is 64 bytes, so two heads
// share each line, and one line of scales serves four tokens of all heads:
// with the hint those shared lines were evicted between their readers (HBM
// fetches 1.68x the cache bytes, measured), with the default policy 1.09x.
template <class C>
constexpr int row_policy() {
  return std::is_same<C, MfmaFP4>::value ? kDefaultPolicy : kStreamPolicy;
}

template <class C, int NB>
__device__ __forceinline__ void row_load_k(const DecodeArgs& p, int g, const int (&id)[NB], int lane,
                                           StepRegs<C, NB>& sr) {
  const KVLayout L = kv_layout<C>(p.flags, p.dims.num_kv_heads);
  const int off = C::k_lane_off(L, g, lane & 15, lane >> 4);
  const int soff = C::k_scale_off(L, g, lane & 15, lane >> 4);
#pragma unroll
  for (int b = 0; b < NB; ++b)
    C::template load_k<row_policy<C>()>(sr.k[b], block_rsrc(p.k_cache, L.block, id[b]), off, L, soff);
}
// FP8 K tiles go through LDS.  A wave's K loads in the MFMA operand layout
// read 16 token rows x 64 bytes per instruction; loads that read whole
// 128-byte rows (eight rows per instruction) made the FP8 call ~4% faster
// in a timing-only test, and staging the rows in LDS with direct loads keeps
// that pattern while the operand layout comes from LDS reads (FP8 call
// 119.6-121.2 against 122.7-129.0 us medians on 128 contexts of
// 1024..4096 tokens; bf16 gained nothing from whole-row K loads).  Per wave
// and register set a buffer of NB blocks x 16 rows x 128 bytes: chunk c (16
// bytes) of row n sits in slot 8n + (c ^ (n >> 1)), so the operand reads of
// 16 lanes (rows 0..15, one chunk) fall in 16 different groups of four
// banks.  Load instruction u of a block fills slots 64u .. 64u + 63, one per
// lane: lane l takes row 8u + l / 8, chunk (l % 8) ^ (row >> 1), whole rows
// per eight lanes.
constexpr int kKStageBlock = 16 * 128;  // bytes of one block's K rows of one kv head (FP8)
template <class C, int NB>
__device__ __forceinline__ void row_load_k_lds(const DecodeArgs& p, int g, const int (&id)[NB], int lane,
                                               uint8_t* buf) {
  const KVLayout L = kv_layout<C>(p.flags, p.dims.num_kv_heads);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(p.k_cache, L.block, id[b]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * u + (lane >> 3);
      const int chunk = (lane & 7) ^ (row >> 1);
      kv_load16_lds<row_policy<C>()>(rs, buf + b * kKStageBlock + 1024 * u, row * L.tok + g * L.head + 16 * chunk);
    }
  }
}
// The K operand registers of a step from its LDS buffer: lane (kg, n) takes
// chunks kg and 4 + kg of row n (head-dim 16kg .. 16kg + 15 and 64 more).
template <class C, int NB>
__device__ __forceinline__ void row_read_k_lds(const uint8_t* buf, int lane, StepRegs<C, NB>& sr) {
  const int n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      sr.k[b].k[u] = *reinterpret_cast<const uint4*>(buf + b * kKStageBlock + 16 * (8 * n + ((4 * u + kg) ^ (n >> 1))));
}

template <class C, int NB>
__device__ __forceinline__ void row_load_v(const DecodeArgs& p, int g, const int (&id)[NB], int lane,
                                           StepRegs<C, NB>& sr) {
  const KVLayout L = kv_layout<C>(p.flags, p.dims.num_kv_heads);
  const int off = C::v_lane_off(L, g, lane & 15, lane >> 4);
  const int soff = C::v_scale_off(L, g, lane & 15, lane >> 4);
#pragma unroll
  for (int b = 0; b < NB; ++b)
    C::template load_v<row_policy<C>()>(sr.v[b], block_rsrc(p.v_cache, L.block, id[b]), off, L, soff);
}

// Stages one head's result of a segment in LDS: its accumulators (acc[i][j]
// holds O[row 4kg + j][8n + i], rows 0 .. G - 1 of local kv head hl), the
// rounded-probability sums (psum[j] of lane group kg: row 4kg + j), and the
// fp32 sum and reference of head n (lane n).  No lane exchange is needed.
template <int G, int HG, int SL>
__device__ __forceinline__ void stage_head(RowsSmem<G, HG, SL>& sm, int s, int hl, const WaveState& st, int lane) {
  const int n = lane & 15, kg = lane >> 4;
  const float lsum_e = sum4(st.lsum_e);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * kg + j;
    if (row < G) {
      float* dst = &sm.out[s][hl * G + row][8 * n];
      *reinterpret_cast<float4*>(dst) = make_float4(st.acc[0][j], st.acc[1][j], st.acc[2][j], st.acc[3][j]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(st.acc[4][j], st.acc[5][j], st.acc[6][j], st.acc[7][j]);
      if (n == 0) sm.psum[s][hl * G + row] = st.psum[j];
    }
  }
  if (kg == 0 && n < G) {
    sm.le[s][hl * G + n] = lsum_e;
    sm.ms[s][hl * G + n] = st.ms;
  }
}

// Result stores of the whole-row kernel (outputs and records), with the
// non-temporal hint: nothing in this launch reads them back, and fewer dirty
// lines are left for the end of the kernel.  Call medians (three alternating
// runs): C3 186.2 -> 185.0 us, C5 118.8 -> 117.9 us, FP4 101.0 -> 99.5 us.
// Partition records keep plain stores: with the hint lse_merge took 12.1
// instead of 9.0 us on 4 x 131072 tokens (16.8 MB of records).
#ifndef LGM_ROWS_NT_STORES
#define LGM_ROWS_NT_STORES 1
#endif
__device__ __forceinline__ void res_store(float* p, float v) {
  if constexpr (LGM_ROWS_NT_STORES) __builtin_nontemporal_store(v, p);
  else *p = v;
}
__device__ __forceinline__ void res_store(float4* p, const float4& v) {
  using V = float __attribute__((ext_vector_type(4)));
  if constexpr (LGM_ROWS_NT_STORES) __builtin_nontemporal_store(__builtin_bit_cast(V, v), reinterpret_cast<V*>(p));
  else *p = v;
}
__device__ __forceinline__ void res_store(uint4* p, const uint4& v) {
  using V = unsigned int __attribute__((ext_vector_type(4)));
  if constexpr (LGM_ROWS_NT_STORES) __builtin_nontemporal_store(__builtin_bit_cast(V, v), reinterpret_cast<V*>(p));
  else *p = v;
}

// Writes a batch's staged results, one wave per segment: each of its
// HG * G rows is normalised (scaled by vscale / the rounded-probability sum;
// LSE = ms + log2(le), in natural log) and goes to the final output (bf16)
// and out_lse when the segment is its whole stream, else to its record: a
// split-K partition record ([B][Hq][P][D], [B][Hq][P]) in partition mode, or
// the range's record slot.  Eight columns per lane; a wave reads all its
// rows of a pass from LDS before it stores any.  With SL token slices per
// head a row's SL partial results (each relative to its own reference ms)
// are first combined by log-sum-exp weights 2^(ms_i - max ms); a slice that
// saw no token (le = 0) weighs nothing.
template <class C, int G, int HG, int SL, int NT>
__device__ __forceinline__ void flush_batch(const DecodeArgs& p, const RowsArgs& r, const RowsSmem<G, HG, SL>& sm,
                                            int nseg, int wave, int lane) {
  constexpr int kRows = HG * G;
  constexpr int kCh = kD / 8;
  constexpr int kItems = kRows * kCh;               // 8-column pieces per segment
  constexpr int kPass = 8 / SL;                     // pieces per lane per pass
  constexpr int kPerPass = kPass * kWaveSize;
  for (int s = wave; s < nseg; s += NT / kWaveSize) {
    const SegDesc d = read_seg(sm, s);
    for (int i0 = 0; i0 < kItems; i0 += kPerPass) {
      float4 v0[kPass], v1[kPass];
      float L[kPass], Le[kPass], M[kPass], vsc[kPass];
#pragma unroll
      for (int k = 0; k < kPass; ++k) {
        const int i = i0 + k * kWaveSize + lane;
        const int row = (i < kItems ? i : 0) / kCh, c = (i < kItems ? i : 0) % kCh;
        if constexpr (SL == 1) {
          v0[k] = *reinterpret_cast<const float4*>(&sm.out[s][row][8 * c]);
          v1[k] = *reinterpret_cast<const float4*>(&sm.out[s][row][8 * c + 4]);
          L[k] = sm.psum[s][row];
          Le[k] = sm.le[s][row];
          M[k] = sm.ms[s][row];
        } else {
          float le[SL], ms[SL], mx = -INFINITY;
#pragma unroll
          for (int q = 0; q < SL; ++q) {
            le[q] = sm.le[s][q * kRows + row];
            ms[q] = sm.ms[s][q * kRows + row];
            if (le[q] > 0.f) mx = fmaxf(mx, ms[q]);
          }
          float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
          float ps = 0.f, ls = 0.f;
#pragma unroll
          for (int q = 0; q < SL; ++q) {
            const float w = le[q] > 0.f ? fast_exp2(ms[q] - mx) : 0.f;
            const float4 x0 = *reinterpret_cast<const float4*>(&sm.out[s][q * kRows + row][8 * c]);
            const float4 x1 = *reinterpret_cast<const float4*>(&sm.out[s][q * kRows + row][8 * c + 4]);
            a0 = make_float4(fmaf(w, x0.x, a0.x), fmaf(w, x0.y, a0.y), fmaf(w, x0.z, a0.z), fmaf(w, x0.w, a0.w));
            a1 = make_float4(fmaf(w, x1.x, a1.x), fmaf(w, x1.y, a1.y), fmaf(w, x1.z, a1.z), fmaf(w, x1.w, a1.w));
            ps = fmaf(w, sm.psum[s][q * kRows + row], ps);
            ls = fmaf(w, le[q], ls);
          }
          v0[k] = a0;
          v1[k] = a1;
          L[k] = ps;
          Le[k] = ls;
          M[k] = mx;
        }
        vsc[k] = C::kFp8 ? sm.vscale[s][row / G] : 1.f;
      }
#pragma unroll
      for (int k = 0; k < kPass; ++k) {
        const int i = i0 + k * kWaveSize + lane;
        if (i >= kItems) continue;
        const int row = i / kCh, c = i % kCh;
        const float inv = L[k] > 0.f ? vsc[k] / L[k] : 0.f;
        const float4 a = make_float4(v0[k].x * inv, v0[k].y * inv, v0[k].z * inv, v0[k].w * inv);
        const float4 b = make_float4(v1[k].x * inv, v1[k].y * inv, v1[k].z * inv, v1[k].w * inv);
        const float ls = Le[k] > 0.f ? (M[k] + fast_log2(Le[k])) * kLn2 : -INFINITY;
        const int64_t orow = (int64_t)d.b * p.dims.num_q_heads + (int64_t)d.hg * kRows + row;
        if (d.whole) {
          const uint32_t w0 = (uint32_t)f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
          const uint32_t w2 = (uint32_t)f32_to_bf16_rne(b.x) | ((uint32_t)f32_to_bf16_rne(b.y) << 16);
          const uint32_t w3 = (uint32_t)f32_to_bf16_rne(b.z) | ((uint32_t)f32_to_bf16_rne(b.w) << 16);
          res_store(reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow * kD + 8 * c),
                    make_uint4(w0, w1, w2, w3));
          if (c == 0 && p.out_lse) res_store(p.out_lse + orow, ls);
        } else if (r.part_tiles > 0) {
          const int64_t prow = orow * p.max_partitions + d.rec;
          float* dst = p.part_out + prow * kD + 8 * c;  // plain stores: lse_merge reads them next, from the caches
          *reinterpret_cast<float4*>(dst) = a;
          *reinterpret_cast<float4*>(dst + 4) = b;
          if (c == 0) p.part_lse[prow] = ls;
        } else {
          float* dst = r.rec_out + ((int64_t)d.rec * kRows + row) * kD + 8 * c;
          res_store(reinterpret_cast<float4*>(dst), a);
          res_store(reinterpret_cast<float4*>(dst + 4), b);
          if (c == 0) res_store(r.rec_lse + (int64_t)d.rec * kRows + row, ls);
        }
      }
    }
  }
}

// Register sets per wave: how many (step, head) pairs of loads a wave keeps
// in flight.  Two cover HBM latency at one wave per SIMD (a bf16 set holds
// 16 KB of one kv head's K and V, an FP8 set 8 KB; more sets or larger steps
// gave FP8 no more bandwidth, see step_blocks).
#ifndef LGM_ROW_SETS_BF16
#define LGM_ROW_SETS_BF16 2
#endif
#ifndef LGM_ROW_SETS_FP8
#define LGM_ROW_SETS_FP8 2
#endif
#ifndef LGM_ROW_SETS_FP4
#define LGM_ROW_SETS_FP4 2
#endif
template <class C>
constexpr int row_sets() {
  return std::is_same<C, MfmaFP8>::value ? LGM_ROW_SETS_FP8
                                         : (std::is_same<C, MfmaFP4>::value ? LGM_ROW_SETS_FP4 : LGM_ROW_SETS_BF16);
}

template <class SM>
__device__ __forceinline__ SegDesc read_seg(const SM& sm, int s) {
  SegDesc d;
  d.b = __builtin_amdgcn_readfirstlane(sm.seg[s].b);
  d.ctx = __builtin_amdgcn_readfirstlane(sm.seg[s].ctx);
  d.lt = __builtin_amdgcn_readfirstlane(sm.seg[s].lt);
  d.et = __builtin_amdgcn_readfirstlane(sm.seg[s].et);
  d.hg = __builtin_amdgcn_readfirstlane(sm.seg[s].hg);
  d.rec = __builtin_amdgcn_readfirstlane(sm.seg[s].rec);
  d.whole = __builtin_amdgcn_readfirstlane(sm.seg[s].whole);
  d.pad = 0;
  return d;
}

// The workgroup stages a batch of nseg segments (descriptors already in
// sm.seg), one wave per segment: the first kStageWin windows of the
// segment's block ids, its query rows and, for FP8, the head group's K and V
// scales.  A wave issues all its loads before it stores any of them to LDS,
// so the batch costs one memory round trip.
template <class C, int G, int HG, int SL, int NT>
__device__ __forceinline__ void stage_batch(const DecodeArgs& p, RowsSmem<G, HG, SL>& sm, int nseg, int wave,
                                            int lane) {
  constexpr int kIdsPer = kStageWin * 2 * kWin / kWaveSize;  // ids per lane
  constexpr int kRows = HG * G;
  constexpr int kQCh = kRows * (kD / 8);                     // 16-byte query chunks per segment
  constexpr int kQPass = 8;                                  // chunks per lane per pass
  const int MB = p.dims.max_blocks_per_seq;
  const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
  for (int s = wave; s < nseg; s += NT / kWaveSize) {
    const SegDesc d = read_seg(sm, s);
    const int lb_end = (d.ctx + kBS - 1) / kBS;  // <= MB: contexts are clamped to the table's capacity
    const int32_t* bt = p.block_tables + (int64_t)d.b * MB;
    int idv[kIdsPer];
#pragma unroll
    for (int k = 0; k < kIdsPer; ++k) {
      const int e = k * kWaveSize + lane;
      const int tile = d.lt + (e >> 1);
      const int lb = 2 * tile + (e & 1);
      idv[k] = (tile < d.et && lb < lb_end) ? bt[lb] : -1;
    }
    float ks = 1.f, vs = 1.f;
    if constexpr (C::kFp8) {
      if (lane < HG) {
        ks = kv_scale(p.k_scale, p.flags, d.hg * HG + lane);
        vs = kv_scale(p.v_scale, p.flags, d.hg * HG + lane);
      }
    }
    const uint16_t* qbase = static_cast<const uint16_t*>(p.q) + (int64_t)d.b * p.q_seq_stride + (int64_t)d.hg * kRows * kD;
    for (int c0 = 0; c0 < kQCh; c0 += kQPass * kWaveSize) {
      uint4 qv[kQPass];
#pragma unroll
      for (int k = 0; k < kQPass; ++k) {
        const int c = c0 + k * kWaveSize + lane;
        qv[k] = make_uint4(0, 0, 0, 0);
        if (c < kQCh) {
          const uint16_t* src = qbase + (c / (kD / 8)) * kD + 8 * (c % (kD / 8));
          if (qvec) {
            qv[k] = *reinterpret_cast<const uint4*>(src);
          } else {
            uint32_t w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = (uint32_t)src[2 * t] | ((uint32_t)src[2 * t + 1] << 16);
            qv[k] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kQPass; ++k) {
        const int c = c0 + k * kWaveSize + lane;
        if (c < kQCh) *reinterpret_cast<uint4*>(&sm.q[s][c / (kD / 8)][8 * (c % (kD / 8))]) = qv[k];
      }
    }
#pragma unroll
    for (int k = 0; k < kIdsPer; ++k) {
      const int e = k * kWaveSize + lane;
      const int id = idv[k];
      sm.ids[s][e / (2 * kWin)][e % (2 * kWin)] = (unsigned)id < (unsigned)p.dims.num_blocks ? id : -1;
    }
    if constexpr (C::kFp8) {
      if (lane < HG) {
        sm.kscale[s][lane] = ks;
        sm.vscale[s][lane] = vs;
      }
    }
  }
}

// Query rows of kv head `hl` (inside the head group) of staged segment s as
// the B operand of the score MFMAs (zero for n >= G).
template <class C, int G, int HG, int SL>
__device__ __forceinline__ void lds_q_operand(const RowsSmem<G, HG, SL>& sm, int s, int hl, short8 (&qb)[4], int n,
                                              int kg) {
  const uint16_t* row = sm.q[s][hl * G + (n < G ? n : 0)];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = *reinterpret_cast<const uint4*>(row + score_d<C>(c, kg, 0));
    if (n >= G) v = make_uint4(0, 0, 0, 0);
    qb[c] = __builtin_bit_cast(short8, v);
  }
}

// One wave's work on a batch of segments: a continuous pipeline over the
// sequence of (step, head) pairs of all the batch's segments, in steps of NB
// 16-token blocks (NB / 2 tiles).  The wave owns kv heads wave * HPW ..
// + HPW - 1 of each segment's head group.  NS register sets hold pairs
// j, j + NS, j + 2NS, ...: a set's next pair is loaded as soon as its
// current one's MFMAs have consumed the registers (K after the scores, V
// after P V), and when the next pair lies in the next segment its loads go
// out before the current segment ends, so moving to a new segment costs no
// wait for memory.  A load cursor runs NS / HPW steps ahead of the compute
// cursor; block ids come from the staged first window of a segment, later
// windows are read from the table one window ahead.  At each segment's end
// the wave writes its heads' results and takes the next segment's query rows
// from LDS.  Segments without tiles (empty contexts) write out = 0 and
// lse = -inf.  Pairs past the batch are absent: their loads return zeros
// without touching memory.
template <class C, int G, int HG, int HPW, int SL>
__device__ __forceinline__ void run_batch(const DecodeArgs& p, RowsSmem<G, HG, SL>& sm, int nseg, int wave, int lane,
                                          uint8_t* kst) {
  constexpr int NB = step_blocks<C>();
  constexpr int ST = NB / 2;  // tiles per step
  constexpr int NS = row_sets<C>();
  static_assert(NS % HPW == 0, "a set must stay on one head");
  static_assert(kWin % ST == 0 && SL * ST <= kWin, "a step's tiles share one window of block ids");
  static_assert(SL == 1 || HPW == 1, "token slices take one head per wave");
  const int n = lane & 15, kg = lane >> 4;
  // The wave's heads (hl0 .. hl0 + HPW - 1 of the group) and its token
  // slice: it takes the segment's steps slice, slice + SL, ...
  const int hl0 = (wave % (HG / HPW)) * HPW;
  const int slice = wave / (HG / HPW);
  auto nsteps_of = [&](int s) {
    const int all = (sm.seg[s].et - sm.seg[s].lt + ST - 1) / ST;
    return __builtin_amdgcn_readfirstlane(all > slice ? (all - slice + SL - 1) / SL : 0);
  };

  // ---- load cursor: segment ls, step lk (ls == nseg: past the batch) ----
  int ls = 0, lk = 0, lwin = 0, l_nsteps = 0, l_b = 0, l_lt = 0, l_et = 0, l_lbend = 0, l_g0 = hl0;
  int lids = -1, lnext = -1;
  // Windows 0 .. kStageWin - 1 come from LDS; a longer segment's later
  // windows are read from the table one window ahead.
  auto l_window = [&](int w) {
    if (w < kStageWin) {
      lids = sm.ids[ls][w][lane];
    } else {
      lids = lnext;
    }
    if (w + 1 >= kStageWin && l_lt + kWin * (w + 1) < l_et)
      lnext = preload_row_ids(p, l_b, l_lt, l_et, l_lbend, kWin * (w + 1), lane);
  };
  auto l_enter = [&](int s) {
    const SegDesc d = read_seg(sm, s);
    ls = s;
    lk = 0;
    lwin = 0;
    l_nsteps = nsteps_of(s);
    l_b = d.b;
    l_lt = d.lt;
    l_et = d.et;
    l_lbend = (d.ctx + kBS - 1) / kBS;
    l_g0 = d.hg * HG + hl0;
    l_window(0);
  };
  auto l_advance = [&]() {
    if (ls >= nseg) return;
    if (++lk < l_nsteps) {
      if ((ST * (slice + SL * lk)) / kWin != lwin) l_window(++lwin);
      return;
    }
    int s = ls + 1;
    while (s < nseg && nsteps_of(s) == 0) ++s;
    if (s < nseg) l_enter(s);
    else ls = nseg;
  };
  auto l_ids = [&](int (&id)[NB]) {
    const int kt = ST * (slice + SL * lk) - kWin * lwin;  // first tile of the step inside its window
#pragma unroll
    for (int t = 0; t < ST; ++t) {
      id[2 * t] = ls < nseg ? __builtin_amdgcn_readlane(lids, 2 * (kt + t)) : -1;
      id[2 * t + 1] = ls < nseg ? __builtin_amdgcn_readlane(lids, 2 * (kt + t) + 1) : -1;
    }
  };
  auto valid_bits = [](const int (&id)[NB]) {
    uint32_t v = 0;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) v |= (id[bb] >= 0 ? 1u : 0u) << bb;
    return v;
  };

  // ---- compute cursor: segment cs, step ck ----
  int cs = 0, ck = 0, c_nsteps = 0, c_lt = 0, c_ctx = 0;
  short8 qb[HPW][4];
  float csc[HPW];
  WaveState st[HPW];
  auto write_empty = [&](int s) {  // a segment without tiles (an empty context): out = 0, lse = -inf
    WaveState e;
    e.reset();
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) stage_head<G, HG, SL>(sm, s, wave * HPW + hh, e, lane);
  };
  auto c_enter = [&](int s) {
    const SegDesc d = read_seg(sm, s);
    cs = s;
    ck = 0;
    c_nsteps = nsteps_of(s);
    c_lt = d.lt;
    c_ctx = d.ctx;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      lds_q_operand<C, G, HG, SL>(sm, s, hl0 + hh, qb[hh], n, kg);
      float c = p.softmax_scale * kLog2e;
      if constexpr (C::kFp8) c *= sm.kscale[s][hl0 + hh];
      csc[hh] = fold_score_scale(c, qb[hh]);
      st[hh].reset();
    }
  };
  int s0 = 0;
  while (s0 < nseg && nsteps_of(s0) == 0) write_empty(s0++);
  if (s0 >= nseg) return;
  c_enter(s0);
  l_enter(s0);

  StepRegs<C, NB> sr[NS];
  int pid[NS][NB];
#pragma unroll
  for (int j = 0; j < NS; ++j) {  // the loop's load order: K, V of each set in turn
    if (j % HPW == 0 && j > 0) l_advance();
    l_ids(pid[j]);
    if constexpr (C::kFp8) row_load_k_lds<C, NB>(p, l_g0 + j % HPW, pid[j], lane, kst + j * NB * kKStageBlock);
    else row_load_k<C, NB>(p, l_g0 + j % HPW, pid[j], lane, sr[j]);
    __builtin_amdgcn_sched_barrier(0);
    row_load_v<C, NB>(p, l_g0 + j % HPW, pid[j], lane, sr[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  bool done = false;
  while (!done) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int h = j % HPW;
      if (j > 0 && done) break;  // (one head per wave: the batch may end between two sets)
      if (h == 0) l_advance();
      int nid[NB];
      l_ids(nid);
      const int lg = l_g0 + h;
      float4v sc[NB];
      if constexpr (C::kFp8) row_read_k_lds<C, NB>(kst + j * NB * kKStageBlock, lane, sr[j]);
      step_scores<C, NB>(sr[j], qb[h], sc);
      if constexpr (C::kFp8) {
        // The buffer's reads are complete before the next step's loads may
        // write it (a load of an absent block lands in LDS at once), and no
        // memory access moves across this point.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        row_load_k_lds<C, NB>(p, lg, nid, lane, kst + j * NB * kKStageBlock);
      } else {
        row_load_k<C, NB>(p, lg, nid, lane, sr[j]);
      }
      step_update<C, NB>(st[h], sr[j], sc, csc[h], valid_bits(pid[j]), kTile * (c_lt + ST * (slice + SL * ck)),
                         c_ctx, kg);
      row_load_v<C, NB>(p, lg, nid, lane, sr[j]);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) pid[j][bb] = nid[bb];
      if (h == HPW - 1 && ++ck == c_nsteps) {  // the segment is done: write it, move to the next
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) stage_head<G, HG, SL>(sm, cs, wave * HPW + hh, st[hh], lane);
        int s = cs + 1;
        while (s < nseg && nsteps_of(s) == 0) write_empty(s++);
        if (s >= nseg) done = true;
        else c_enter(s);
      }
    }
  }
  // The K loads issued past the batch's last step (absent blocks) may still
  // be in flight; the next batch's first loads fill the same buffers, and
  // nothing orders two loads' arrival in LDS, so they complete here.
  if constexpr (C::kFp8) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A segment costs its workgroup more than its tiles (entering it, staging its
// query and writing its result), so ranges are cut in equal cost: kTileCost
// per tile plus seg_cost<C>() per stream.  Measured with per-workgroup
// timestamps on equal tile ranges: 128 FP8 contexts of 1024..4096 tokens,
// ranges holding two segments ended 3-5 us after ranges holding one (a
// range takes ~100 us; 8% of the workgroups' time idle at the end); bf16
// (64 contexts of 512..8192): ~1 us.  FP8 call medians by the cost per
// stream (quarter tiles): 0: 119.0-120.4 us, 3: 117.3-118.1, 6: 116.8-117.4,
// 10: 116.5-116.7 (16: slower again); bf16 and FP4 moved within noise.
constexpr int kTileCost = 4;
#ifndef LGM_ROWS_SEG_COST_BF16
#define LGM_ROWS_SEG_COST_BF16 1
#endif
#ifndef LGM_ROWS_SEG_COST_FP8
#define LGM_ROWS_SEG_COST_FP8 10
#endif
#ifndef LGM_ROWS_SEG_COST_FP4
#define LGM_ROWS_SEG_COST_FP4 4
#endif
static_assert(kTileCost == 4 && LGM_ROWS_SEG_COST_BF16 <= 16 && LGM_ROWS_SEG_COST_FP8 <= 16 &&
                  LGM_ROWS_SEG_COST_FP4 <= 16,
              "the host checks the total cost against 4 per tile and 16 * 8 per stream");
template <class C>
constexpr int seg_cost() {
  return std::is_same<C, MfmaFP8>::value ? LGM_ROWS_SEG_COST_FP8
                                         : (std::is_same<C, MfmaFP4>::value ? LGM_ROWS_SEG_COST_FP4 : LGM_ROWS_SEG_COST_BF16);
}

// One workgroup per equal range of the flattened list of work units: the
// 32-token tiles of all streams, or (partition mode) their split-K
// partitions, so that a range holds whole partitions.  Record slot 2w holds
// range w's first stream when split, slot 2w + 1 its last one (when that is
// another stream); so piece k >= 1 of a split stream, held by workgroup
// i0 + k where it is the first stream, is in slot 2(i0 + k), and only its
// first piece's slot needs recording: wg_first[u] = that slot, wg_last[u] =
// the workgroup holding the stream's last tile.  An empty range (more
// workgroups than tiles) writes LSE -inf in slot 2w, so a stream that spans
// it merges a record of weight zero there.  In partition mode every
// partition of a split context writes its own record, at its index.  The
// range's segments are located, staged and run in batches.
template <class C, int G, int HPW, int NT, int SL = 1>
__global__ __launch_bounds__(NT, 1) void paged_decode_rows_kernel(DecodeArgs p, RowsArgs r) {
  constexpr int HG = NT / kWaveSize * HPW / SL;
  static_assert(HG * SL == NT / kWaveSize * HPW, "whole waves per token slice");
  using Bt = Batch<G, HG, SL>;
  __shared__ RowsSmem<G, HG, SL> sm;
  constexpr int kKStage = C::kFp8 ? row_sets<C>() * step_blocks<C>() * kKStageBlock : 0;  // per wave
  __shared__ __attribute__((aligned(16))) uint8_t kst[kKStage > 0 ? NT / kWaveSize * kKStage : 16];
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int B = p.dims.num_seqs;
  const int nhg = p.dims.num_kv_heads / HG;
  const int W = gridDim.x;
  const int wg = blockIdx.x;
  const bool parts = r.part_tiles > 0;
  const int upt = parts ? r.part_tiles : 1;   // tiles per unit
  const int unit = kTile * upt;               // tokens per unit
  const int min_units = 1;                    // an empty context still writes out = 0, lse = -inf
  // Equal ranges of cost: kTileCost per tile and seg_cost<C>() per stream
  // (partition mode: one per partition).
  const int ucost = parts ? 1 : kTileCost;
  // A tile of a smaller head group carries fewer bytes while entering and
  // writing a segment costs about the same, so the per-stream cost grows as
  // 8 / HG (1 kv head, G = 8, FP8, 1024 contexts: 130.9 -> 126.6 us; 1 and
  // 2 kv heads in bf16 and FP4 1-3% faster).
  const int scost = parts ? 0 : seg_cost<C>() * (8 / HG);

  int total = scan_chunk<NT>(p, sm, 0, nhg, unit, min_units, ucost, scost);
  for (int c0 = kChunk; c0 < B; c0 += kChunk) total += scan_chunk<NT>(p, sm, c0, nhg, unit, min_units, ucost, scost);
  const int t_lo = (int)((int64_t)wg * total / W);
  const int t_hi = (int)((int64_t)(wg + 1) * total / W);
  int b0 = 0, base = 0;
  if (B > kChunk) scan_chunk<NT>(p, sm, 0, nhg, unit, min_units, ucost, scost);  // back to the first chunk

  int pos = t_lo;
  bool first = true;
  while (pos < t_hi) {
    int nseg = 0;
    while (pos < t_hi && nseg < Bt::kMax) {
      int rel = pos - base;
      while (rel >= __builtin_amdgcn_readfirstlane(sm.pre[kChunk])) {  // uniform: every thread moves on together
        base += __builtin_amdgcn_readfirstlane(sm.pre[kChunk]);
        b0 += kChunk;
        scan_chunk<NT>(p, sm, b0, nhg, unit, min_units, ucost, scost);
        rel = pos - base;
      }
      int lo = 0, hi = kChunk;  // sm.pre[lo] <= rel < sm.pre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(sm.pre[mid]) <= rel) lo = mid;
        else hi = mid;
      }
      const int b = b0 + lo;
      const int ctx = __builtin_amdgcn_readfirstlane(clamped_ctx(p, b));
      const int ntb = (ctx + kTile - 1) / kTile;                      // tiles of the stream
      const int ntu = max((ctx + unit - 1) / unit, min_units);        // units of the stream
      const int off = rel - __builtin_amdgcn_readfirstlane(sm.pre[lo]);
      const int stream_cost = scost + ucost * ntu;
      const int hg = off / stream_cost;
      // The range holds the units whose cost position scost + ucost * j
      // (the unit's start) lies in [c0, c1), its part of this stream.
      const int c0 = off - hg * stream_cost;
      const int c1 = min(stream_cost, c0 + (t_hi - pos));
      const int lu = c0 <= scost ? 0 : (c0 - scost + ucost - 1) / ucost;
      const int eu = parts ? lu + 1 : (c1 <= scost ? 0 : min(ntu, (c1 - scost + ucost - 1) / ucost));
      pos += parts ? 1 : c1 - c0;
      if (lu >= eu) continue;  // only the stream's fixed cost lies in the range
      const int lt = lu * upt;
      const int et = min(ntb, eu * upt);
      const int u = b * nhg + hg;
      const bool whole = parts ? ntu == 1 : (lu == 0 && eu == ntu);
      if (threadIdx.x == 0) {
        if (!parts) {
          if (lt == 0) r.wg_first[u] = 2 * wg + (first ? 0 : 1);  // the record slot of the stream's first piece
          if (et == ntb) r.wg_last[u] = wg;
        }
        sm.seg[nseg] = SegDesc{b, ctx, lt, et, hg, parts ? lu : 2 * wg + (first ? 0 : 1), whole ? 1 : 0, 0};
      }
      first = false;
      ++nseg;
    }
    __syncthreads();  // the batch's descriptors
    stage_batch<C, G, HG, SL, NT>(p, sm, nseg, wave, lane);
    __syncthreads();  // the batch's ids, query rows and scales
    run_batch<C, G, HG, HPW, SL>(p, sm, nseg, wave, lane, kst + wave * kKStage);
    __syncthreads();  // every wave has staged its results
    flush_batch<C, G, HG, SL, NT>(p, r, sm, nseg, wave, lane);
    __syncthreads();  // the batch is written before the next one is staged
  }
  // A range without a unit (more workgroups than units, or only streams'
  // fixed costs): its first record slot weighs nothing in the merge of a
  // stream it lies inside.
  if (!parts && first) {
    for (int i = threadIdx.x; i < HG * G; i += NT) r.rec_lse[(int64_t)2 * wg * HG * G + i] = -INFINITY;
  }
}

// Log-sum-exp merge of the records of split streams (the combine step of the
// split-K method; [mainarch] decode attention, [Loom] local split-K/LSE
// merge).  One workgroup per (sequence, query head); streams written whole
// by the decode kernel are skipped, empty contexts get out = 0, lse = -inf.
// Four rows per workgroup: the merge kernel's average over C3, C5 and the
// FP4 workload was 5.92 us, against 6.17 us with one row and 6.29 us with 16.
#ifndef LGM_ROWS_MERGE_THREADS
#define LGM_ROWS_MERGE_THREADS 256
#endif
constexpr int kMergeThreads = LGM_ROWS_MERGE_THREADS;
constexpr int kMergeRows = kMergeThreads / kWaveSize;  // one wave per (sequence, query head) row
constexpr int kMergeLanes = kD / 8;                    // lanes per record row: eight columns each
constexpr int kMergeGroups = kWaveSize / kMergeLanes;  // records in flight per wave

// Merge of the records of one output row: two memory round trips.  The
// first reads the row's context length and its stream's first record slot
// and last workgroup; the second reads, together, the LSE of every piece
// (lane k holds piece k) and the records of the first 8 pieces (the wave
// works as four groups of 16 lanes, group q holding pieces q, q + 4, ...,
// eight columns per lane).  Max and sum are lane shuffles, the groups' sums
// are added by lane shuffles at the end: no LDS, no barrier.  Streams of
// more pieces read the rest in a further pass.
__global__ __launch_bounds__(kMergeThreads) void rows_merge_kernel(DecodeArgs p, RowsArgs r) {
  // Pieces per group read with the LSEs.  Two (the first 8 pieces) keep the
  // kernel at 48 VGPRs, 8 waves per SIMD; four took 66 VGPRs (7 waves), and
  // rows past what fits waited for a second round.  Merge times (rocprofv3,
  // C3 / C5 / FP8 and bf16 at G = 8): 4.62 / 6.03 / 8.86 / 5.91 us with two,
  // 5.16 / 6.48 / 10.22 / 6.36 with four, 5.32 / 5.81 / 8.26 / 6.16 with one.
#ifndef LGM_ROWS_MERGE_PRE
#define LGM_ROWS_MERGE_PRE 2
#endif
  constexpr int kPre = LGM_ROWS_MERGE_PRE;
  const int lane = threadIdx.x % kWaveSize;
  const int Hq = p.dims.num_q_heads;
  const int orow = blockIdx.x * kMergeRows + threadIdx.x / kWaveSize;
  if (orow >= p.dims.num_seqs * Hq) return;
  const int b = orow / Hq;
  const int h = orow - b * Hq;
  const int G = Hq / p.dims.num_kv_heads;
  const int g = h / G;
  const int HG = r.head_group;
  const int nhg = p.dims.num_kv_heads / HG;
  const int u = b * nhg + g / HG;
  // The context length and the stream's slots do not depend on each other:
  // all three loads are issued before any is used.
  const int ctx = clamped_ctx(p, b);
  const int s0 = r.wg_first[u];
  const int i1 = r.wg_last[u];
  uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)orow * kD;
  const int grp = lane / kMergeLanes;
  const int c = lane % kMergeLanes;
  if (ctx == 0) {
    if (grp == 0) *reinterpret_cast<uint4*>(out + 8 * c) = make_uint4(0, 0, 0, 0);
    if (lane == 0 && p.out_lse) p.out_lse[orow] = -INFINITY;
    return;
  }
  const int i0 = s0 >> 1;
  if (i0 == i1) return;  // the only workgroup of the stream wrote the row itself
  const int n = i1 - i0 + 1;
  const int64_t rec_rows = (int64_t)HG * G;
  const int hrow = (g % HG) * G + h % G;
  auto slot = [&](int k) -> int64_t { return k == 0 ? s0 : 2 * (int64_t)(i0 + k); };
  auto lse_of = [&](int k) -> float { return r.rec_lse[slot(k) * rec_rows + hrow]; };
  auto rec_ptr = [&](int k) -> const float4* {
    return reinterpret_cast<const float4*>(r.rec_out + (slot(k) * rec_rows + hrow) * kD) + 2 * c;
  };

  const float ls0 = lane < n ? lse_of(lane) : -INFINITY;
  float4 pa[kPre], pb[kPre];
#pragma unroll
  for (int m = 0; m < kPre; ++m) {
    const int k = grp + kMergeGroups * m;
    const float4* src = rec_ptr(k < n ? k : 0);
    pa[m] = src[0];
    pb[m] = src[1];
  }
  float mx = ls0;
  for (int k = lane + kWaveSize; k < n; k += kWaveSize) mx = fmaxf(mx, lse_of(k));
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float ms = mx == -INFINITY ? 0.f : mx;
  const float w0 = ls0 == -INFINITY ? 0.f : expf(ls0 - ms);
  float sw = w0;
  for (int k = lane + kWaveSize; k < n; k += kWaveSize) {
    const float l = lse_of(k);
    sw += l == -INFINITY ? 0.f : expf(l - ms);
  }
  const float S = group_sum<kWaveSize>(sw);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // A piece of weight zero (an empty range, or past the stream) is left out
  // by a select, so its record's bytes never reach the sum.
  auto fold = [&](float wk, const float4& v0, const float4& v1) {
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wk == 0.f ? acc[e] : fmaf(wk, x[e], acc[e]);
  };
#pragma unroll
  for (int m = 0; m < kPre; ++m) {
    const int k = grp + kMergeGroups * m;  // below 64: lanes at or past n have weight 0
    const float wk = __shfl(w0, k);        // every lane takes part in the shuffle
    fold(k < n ? wk : 0.f, pa[m], pb[m]);
  }
  for (int k0 = kMergeGroups * kPre; k0 < n; k0 += kMergeGroups) {  // n is the same across the wave
    const int k = k0 + grp;
    const float wl = __shfl(w0, k % kWaveSize);
    float wk = 0.f;
    if (k < n) {
      if (k < kWaveSize) {
        wk = wl;
      } else {
        const float l = lse_of(k);
        wk = l == -INFINITY ? 0.f : expf(l - ms);
      }
    }
    const float4* src = rec_ptr(k < n ? k : 0);
    fold(wk, src[0], src[1]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], kMergeLanes);
    acc[e] += __shfl_xor(acc[e], 2 * kMergeLanes);
  }
  if (grp == 0) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = S > 0.f ? acc[2 * e] / S : 0.f;
      const float bb = S > 0.f ? acc[2 * e + 1] / S : 0.f;
      o[e] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(bb) << 16);
    }
    *reinterpret_cast<uint4*>(out + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0 && p.out_lse) p.out_lse[orow] = S > 0.f ? mx + logf(S) : -INFINITY;
}

// Workgroup shape for a head group of 8: four waves of two heads (one wave
// per SIMD), except for FP4, which runs eight waves of one head, two per SIMD,
// each within half the register file.  FP4 moves the fewest bytes per
// instruction; with one wave per SIMD its dependency stalls were exposed, and
// eight waves made it ~10% faster, while FP8 was ~2% slower with eight.
// Groups of more than 11 query heads would not fit half the register file
// (the eight-wave build spills 8 to 92 bytes per lane to scratch memory at
// G = 12..16) and keep four waves of two heads, should the head groups of 8
// be widened past LGM_ROWS_HG8_MAX_GROUP.
#ifndef LGM_FP4_EIGHT_WAVES
#define LGM_FP4_EIGHT_WAVES 1
#endif
constexpr int kEightWaveMaxGroup = 11;
template <class C, int G>
constexpr bool two_waves_per_simd() {
  return LGM_FP4_EIGHT_WAVES && std::is_same<C, MfmaFP4>::value && G <= kEightWaveMaxGroup;
}

template <class C, int G>
hipError_t launch_group(const DecodeArgs& a, const RowsArgs& r, hipStream_t s) {
  if (r.head_group == 8) {
    if constexpr (G > LGM_ROWS_HG8_MAX_GROUP)
      return hipErrorInvalidValue;  // the planner takes groups of 4 kv heads there
    else if constexpr (two_waves_per_simd<C, G>())
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, 2 * kDecodeThreads>), dim3(r.num_wg),
                         dim3(2 * kDecodeThreads), 0, s, a, r);
    else
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 2, kDecodeThreads>), dim3(r.num_wg), dim3(kDecodeThreads),
                         0, s, a, r);
  } else if (r.head_group == 4) {  // FP4: two token slices per head over eight waves (at G = 9, 10 that
                                   // shape spilled to scratch)
    if constexpr (two_waves_per_simd<C, G>() && G <= 8)
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, 2 * kDecodeThreads, 2>), dim3(r.num_wg),
                         dim3(2 * kDecodeThreads), 0, s, a, r);
    else
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, kDecodeThreads>), dim3(r.num_wg), dim3(kDecodeThreads),
                         0, s, a, r);
  } else if (r.head_group == 2) {  // two token slices per head (FP4: four, over eight waves)
    if constexpr (two_waves_per_simd<C, G>())
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, 2 * kDecodeThreads, 4>), dim3(r.num_wg),
                         dim3(2 * kDecodeThreads), 0, s, a, r);
    else
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, kDecodeThreads, 2>), dim3(r.num_wg), dim3(kDecodeThreads),
                         0, s, a, r);
  } else if (r.head_group == 1) {  // four token slices (FP4: eight)
    if constexpr (two_waves_per_simd<C, G>())
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, 2 * kDecodeThreads, 8>), dim3(r.num_wg),
                         dim3(2 * kDecodeThreads), 0, s, a, r);
    else
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, kDecodeThreads, 4>), dim3(r.num_wg), dim3(kDecodeThreads),
                         0, s, a, r);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || r.part_tiles > 0) return e;  // partition records are merged by lse_merge
  // Short contexts: when every context fits one tile, no stream is split
  // (each, an empty one included, is one unit written by the decode kernel),
  // so the call is a single launch.
  if (a.max_context_len <= kTile) return e;
  const int merge_rows = a.dims.num_seqs * a.dims.num_q_heads;
  hipLaunchKernelGGL(rows_merge_kernel, dim3((merge_rows + kMergeRows - 1) / kMergeRows), dim3(kMergeThreads), 0, s, a,
                     r);
  return hipGetLastError();
}

template <class C>
hipError_t dispatch(const DecodeArgs& a, const RowsArgs& r, int G, hipStream_t s) {
  switch (G) {
#define LGM_CASE(GV) \
  case GV:           \
    return launch_group<C, GV>(a, r, s);
    LGM_CASE(1) LGM_CASE(2) LGM_CASE(3) LGM_CASE(4) LGM_CASE(5) LGM_CASE(6) LGM_CASE(7) LGM_CASE(8)
    LGM_CASE(9) LGM_CASE(10) LGM_CASE(11) LGM_CASE(12) LGM_CASE(13) LGM_CASE(14) LGM_CASE(15) LGM_CASE(16)
#undef LGM_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_rows_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int num_kv_heads, int group,
                           int block_size) {
  return decode_mfma_supported(act, cache, head_dim, group, block_size) && num_kv_heads >= 1;
}

hipError_t launch_paged_decode_rows(const DecodeArgs& a, const RowsArgs& r, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, r, G, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, r, G, s);
  if (cache == LGM_FP4_E2M1) return dispatch<MfmaFP4>(a, r, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
