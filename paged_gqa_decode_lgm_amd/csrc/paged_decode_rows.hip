// Paged GQA decode attention over whole KV token rows, for gfx950 matrix
// cores: bf16 activations, bf16, FP8 E4M3 or FP4 E2M1 (E8M0 block scales)
// caches, head_dim 128, block_size 16, a kv head count divisible by 4.
//
// The split-K method of paged_decode.hip (mainarch README, decode-attention
// section; Loom Kernels README, "Attention" row) with the work laid out for
// how HBM serves a paged NHD cache.  A token row holds all kv heads side by
// side (Hkv x 256 bytes for bf16), and a 16-token block is one contiguous
// run of rows.  Workgroups that each read one kv head's 256-byte slice of
// every row leave the rest of each DRAM page to other workgroups at other
// times; here one workgroup covers a group of HG = 8 (or 4) kv heads, its four
// waves taking 2 (or 1) heads each, so the workgroup reads whole rows and
// whole blocks.
//
// The work is the flattened list of 32-token tiles of all streams (a stream
// is one sequence's tiles for one head group), cut into as many equal ranges
// as workgroups run at once: every workgroup reads the same number of bytes
// whatever the mix of context lengths, and there is no queue.  A range covers
// the end of one stream, whole streams, and the start of another; a stream
// that lies inside one range is written directly, the pieces of a split
// stream go to two record slots per workgroup and are merged by log-sum-exp
// afterwards (rows_merge_kernel).  Since each wave owns its heads for the
// whole range, no wave ever waits for another.
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

struct RowsSmem {
  int pre[kChunk + 1];  // tiles of the streams of sequences b0 .. b0 + j - 1
  int wave_sum[kMaxRowWaves];
};

__device__ __forceinline__ int clamped_ctx(const DecodeArgs& p, int b) {
  const int c = p.context_lens[b];
  return c < 0 ? 0 : (c > p.max_context_len ? p.max_context_len : c);
}

// Fills sm.pre for sequences b0 .. b0 + kChunk - 1 (nhg streams of
// ceil(ctx / unit) work units per sequence: 32-token tiles, or partitions;
// an empty context still counts one) and returns the chunk's total.
// Called by every thread of the NT-thread workgroup (it synchronises).
template <int NT>
__device__ int scan_chunk(const DecodeArgs& p, RowsSmem& sm, int b0, int nhg, int unit, int min_units) {
  constexpr int SPT = kChunk / NT;  // sequences per thread
  static_assert(SPT * NT == kChunk && NT / kWaveSize <= kMaxRowWaves, "scan layout");
  const int tid = threadIdx.x, lane = tid & (kWaveSize - 1), wave = tid / kWaveSize;
  int t[SPT], s = 0;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int b = b0 + SPT * tid + k;
    t[k] = b < p.dims.num_seqs ? max((clamped_ctx(p, b) + unit - 1) / unit, min_units) * nhg : 0;
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

// Writes one head's result of a segment: the final output (bf16, normalised)
// when the segment is the whole stream, else a record (fp32 normalised output
// and natural-log LSE).  acc[i][j] holds O[row 4kg + j][8n + i]; the row's
// max and sums sit in lane `row` of the score layout.
template <class C, int G>
__device__ __forceinline__ void write_head(const DecodeArgs& p, const RowsArgs& r, const WaveState& st, int b, int g,
                                           bool whole, int rec, int lane) {
  const int n = lane & 15, kg = lane >> 4;
  const float lsum_e = sum4(st.lsum_e);
  const float vscale = C::kFp8 ? kv_scale(p.v_scale, p.flags, g) : 1.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * kg + j;
    const float L = st.psum[j];  // rounded-probability sum of head `row`
    const float Le = __shfl(lsum_e, row);
    const float ms = __shfl(st.ms, row);
    if (row < G) {
      const float inv = L > 0.f ? vscale / L : 0.f;
      const float lse = Le > 0.f ? (ms + fast_log2(Le)) * kLn2 : -INFINITY;
      const int64_t orow = (int64_t)b * p.dims.num_q_heads + g * G + row;
      if (whole) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = (uint32_t)f32_to_bf16_rne(st.acc[2 * i][j] * inv) |
                 ((uint32_t)f32_to_bf16_rne(st.acc[2 * i + 1][j] * inv) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow * kD + 8 * n) = make_uint4(w[0], w[1], w[2], w[3]);
        if (n == 0 && p.out_lse) p.out_lse[orow] = lse;
      } else if (r.part_tiles > 0) {
        // split-K record of partition `rec`: [B][Hq][P][D] and [B][Hq][P]
        const int64_t prow = orow * p.max_partitions + rec;
        float* dst = p.part_out + prow * kD + 8 * n;
        *reinterpret_cast<float4*>(dst) =
            make_float4(st.acc[0][j] * inv, st.acc[1][j] * inv, st.acc[2][j] * inv, st.acc[3][j] * inv);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(st.acc[4][j] * inv, st.acc[5][j] * inv, st.acc[6][j] * inv, st.acc[7][j] * inv);
        if (n == 0) p.part_lse[prow] = lse;
      } else {
        const int hrow = (g % r.head_group) * G + row;  // row inside the head group
        float* dst = r.rec_out + ((int64_t)rec * r.head_group * G + hrow) * kD + 8 * n;
        *reinterpret_cast<float4*>(dst) =
            make_float4(st.acc[0][j] * inv, st.acc[1][j] * inv, st.acc[2][j] * inv, st.acc[3][j] * inv);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(st.acc[4][j] * inv, st.acc[5][j] * inv, st.acc[6][j] * inv, st.acc[7][j] * inv);
        if (n == 0) r.rec_lse[(int64_t)rec * r.head_group * G + hrow] = lse;
      }
    }
  }
}

// Register sets per wave: how many (step, head) pairs of loads a wave keeps
// in flight.  Two cover HBM latency at one wave per SIMD (a bf16 set holds
// 16 KB of one kv head's K and V, an FP8 set 8 KB; more sets or larger steps
// gave FP8 no more bandwidth, see step_blocks).
constexpr int kRowSets = 2;

// One segment for this wave: tiles lt .. et - 1 of sequence b (context ctx)
// for kv heads g0 .. g0 + HPW - 1, in steps of NB 16-token blocks (NB / 2
// tiles).  The wave walks pairs s = (step s / HPW, head s % HPW) with NS
// register sets: set j always holds pairs j, j + NS, j + 2NS, ... (one head,
// every NS/HPW-th step).  A set's next step is loaded as soon as its current
// step's MFMAs have consumed the registers (K after the scores, V after
// P V), so while one set is computed the other sets' loads and this set's
// next loads are in flight.  Blocks past the segment are absent: their loads
// return zeros without touching memory and the step masks them, so every
// iteration issues the same loads in the same order.
template <class C, int G, int HPW>
__device__ __forceinline__ void run_segment(const DecodeArgs& p, const RowsArgs& r, int b, int ctx, int lt, int et,
                                            int g0, bool whole, int rec, int lane) {
  constexpr int NB = step_blocks<C>();
  constexpr int ST = NB / 2;  // tiles per step
  constexpr int NS = kRowSets;
  static_assert(NS % HPW == 0, "each set must stay on one head");
  static_assert(32 % ST == 0, "a step's tiles share one window of block ids");
  constexpr int kAdvance = NS / HPW;  // steps a set moves per iteration
  const int kg = lane >> 4;
  short8 qb[HPW][4];
  WaveState st[HPW];
  float csc[HPW];
  const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_seq_stride + (int64_t)(g0 + hh) * G * kD;
    load_q_operand<C, G>(qb[hh], qrow, qvec, lane & 15, kg);
    st[hh].reset();
    float c = p.softmax_scale * kLog2e;
    if constexpr (C::kFp8) c *= kv_scale(p.k_scale, p.flags, g0 + hh);
    csc[hh] = fold_score_scale(c, qb[hh]);
  }

  const int lb_end = (ctx + kBS - 1) / kBS;
  int win = 0;
  int ids = preload_row_ids(p, b, lt, et, lb_end, 0, lane);
  // Block ids of step k (-1 when absent), from the 32-tile window of ids.
  auto step_ids = [&](int k, int (&id)[NB]) {
    const int kt = ST * k;
    if ((kt >> 5) != win) {
      win = kt >> 5;
      ids = preload_row_ids(p, b, lt, et, lb_end, 32 * win, lane);
    }
#pragma unroll
    for (int t = 0; t < ST; ++t) {
      id[2 * t] = __builtin_amdgcn_readlane(ids, 2 * ((kt + t) & 31));
      id[2 * t + 1] = __builtin_amdgcn_readlane(ids, 2 * ((kt + t) & 31) + 1);
    }
  };
  auto valid_bits = [](const int (&id)[NB]) {
    uint32_t v = 0;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) v |= (id[bb] >= 0 ? 1u : 0u) << bb;
    return v;
  };
  StepRegs<C, NB> sr[NS];
  int pid[NS][NB];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    if (j % HPW == 0) {
      step_ids(j / HPW, pid[j]);
    } else {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) pid[j][bb] = pid[j - j % HPW][bb];
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {  // the loop's load order: K, V of each set in turn
    row_load_k<C, NB>(p, g0 + j % HPW, pid[j], lane, sr[j]);
    __builtin_amdgcn_sched_barrier(0);
    row_load_v<C, NB>(p, g0 + j % HPW, pid[j], lane, sr[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nsteps = (et - lt + ST - 1) / ST;
  const int iters = (nsteps + kAdvance - 1) / kAdvance;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int h = j % HPW;
      const int k = it * kAdvance + j / HPW;  // this set's step
      int nid[NB];
      if (h == 0) {
        step_ids(k + kAdvance, nid);
      } else {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) nid[bb] = pid[j - h][bb];  // the head-0 set of the same step looked it up
      }
      float4v s[NB];
      step_scores<C, NB>(sr[j], qb[h], s);
      row_load_k<C, NB>(p, g0 + h, nid, lane, sr[j]);
      step_update<C, NB>(st[h], sr[j], s, csc[h], valid_bits(pid[j]), kTile * (lt + ST * k), ctx, kg);
      row_load_v<C, NB>(p, g0 + h, nid, lane, sr[j]);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) pid[j][bb] = nid[bb];
    }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) write_head<C, G>(p, r, st[hh], b, g0 + hh, whole, rec, lane);
}

// One workgroup per equal range of the flattened list of work units: the
// 32-token tiles of all streams, or (partition mode) their split-K
// partitions, so that a range holds whole partitions.  Metadata for the
// range merge: first_stream[w] = the stream the range starts in (-1 if
// empty), wg_first[u] / wg_last[u] = the workgroups holding stream u's first
// and last tiles.  Record slot 2w holds the range's first stream when split,
// slot 2w + 1 its last one (when that is another stream).  In partition mode
// every partition of a split context writes its own record, at its index.
template <class C, int G, int HPW, int NT>
__global__ __launch_bounds__(NT, 1) void paged_decode_rows_kernel(DecodeArgs p, RowsArgs r) {
  __shared__ RowsSmem sm;
  constexpr int HG = NT / kWaveSize * HPW;
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

  int total = scan_chunk<NT>(p, sm, 0, nhg, unit, min_units);
  for (int c0 = kChunk; c0 < B; c0 += kChunk) total += scan_chunk<NT>(p, sm, c0, nhg, unit, min_units);
  const int t_lo = (int)((int64_t)wg * total / W);
  const int t_hi = (int)((int64_t)(wg + 1) * total / W);
  int b0 = 0, base = 0;
  if (B > kChunk) scan_chunk<NT>(p, sm, 0, nhg, unit, min_units);  // back to the first chunk

  int pos = t_lo;
  bool first = true;
  if (!parts && threadIdx.x == 0 && t_lo >= t_hi) r.first_stream[wg] = -1;
  while (pos < t_hi) {
    int rel = pos - base;
    while (rel >= __builtin_amdgcn_readfirstlane(sm.pre[kChunk])) {  // uniform: every thread moves on together
      base += __builtin_amdgcn_readfirstlane(sm.pre[kChunk]);
      b0 += kChunk;
      scan_chunk<NT>(p, sm, b0, nhg, unit, min_units);
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
    const int hg = off / ntu;
    const int lu = off - hg * ntu;
    const int eu = parts ? lu + 1 : min(ntu, lu + (t_hi - pos));
    const int lt = lu * upt;
    const int et = min(ntb, eu * upt);
    const int u = b * nhg + hg;
    const bool whole = parts ? ntu == 1 : (lu == 0 && eu == ntu);
    if (!parts && threadIdx.x == 0) {
      if (first) r.first_stream[wg] = u;
      if (lt == 0) r.wg_first[u] = wg;
      if (et == ntb) r.wg_last[u] = wg;
    }
    run_segment<C, G, HPW>(p, r, b, ctx, lt, et, hg * HG + wave * HPW, whole,
                           parts ? lu : 2 * wg + (first ? 0 : 1), lane);
    pos += eu - lu;
    first = false;
  }
}

// Log-sum-exp merge of the records of split streams (the combine step of the
// split-K method; [mainarch] decode attention, [Loom] local split-K/LSE
// merge).  One workgroup per (sequence, query head); streams written whole
// by the decode kernel are skipped, empty contexts get out = 0, lse = -inf.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = kMergeThreads / kWaveSize;  // one wave per (sequence, query head) row
constexpr int kMergeLanes = kD / 8;                    // lanes per record row: eight columns each
constexpr int kMergeGroups = kWaveSize / kMergeLanes;  // records in flight per wave

// Merge of the records of one output row.  Lane k first holds the record of
// the k-th workgroup of the stream (64 at a time) and its weight
// exp(lse - max); the wave then works as four groups of 16 lanes, each group
// folding every fourth record into eight columns per lane, and the groups are
// summed by lane shuffles at the end: no LDS, no barrier.
__global__ __launch_bounds__(kMergeThreads) void rows_merge_kernel(DecodeArgs p, RowsArgs r) {
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
  // The context length and the stream's workgroup span do not depend on
  // each other: both loads are issued before either is used.
  const int ctx = clamped_ctx(p, b);
  const int i0 = r.wg_first[u];
  const int i1 = r.wg_last[u];
  uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)orow * kD;
  const int grp = lane / kMergeLanes;
  const int c = lane % kMergeLanes;
  if (ctx == 0) {
    if (grp == 0) *reinterpret_cast<uint4*>(out + 8 * c) = make_uint4(0, 0, 0, 0);
    if (lane == 0 && p.out_lse) p.out_lse[orow] = -INFINITY;
    return;
  }
  if (i0 == i1) return;  // the only workgroup of the stream wrote the row itself
  const int n = i1 - i0 + 1;
  const int64_t rec_rows = (int64_t)HG * G;
  const int hrow = (g % HG) * G + h % G;
  // Record of the k-th workgroup from i0, or -1 for a workgroup whose range
  // is empty (there are more workgroups than tiles).
  auto rec_of = [&](int k) -> int {
    const int w = i0 + k;
    const int f = r.first_stream[w];
    return f < 0 ? -1 : 2 * w + (f == u ? 0 : 1);
  };
  auto lse_of = [&](int rec) -> float { return rec < 0 ? -INFINITY : r.rec_lse[rec * rec_rows + hrow]; };

  // The first 64 records stay in registers; longer spans reload the rest.
  const int rc0 = lane < n ? rec_of(lane) : -1;
  const float ls0 = lse_of(rc0);
  float mx = ls0;
  for (int k = lane + kWaveSize; k < n; k += kWaveSize) mx = fmaxf(mx, lse_of(rec_of(k)));
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float ms = mx == -INFINITY ? 0.f : mx;
  const float w0 = rc0 < 0 ? 0.f : expf(ls0 - ms);
  float sw = w0;
  for (int k = lane + kWaveSize; k < n; k += kWaveSize) {
    const int rc = rec_of(k);
    sw += rc < 0 ? 0.f : expf(lse_of(rc) - ms);
  }
  const float S = group_sum<kWaveSize>(sw);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // A record that is absent reads record 0 (always in the workspace) and is
  // dropped by a select, so unwritten workspace bytes never reach the sum.
  auto fold = [&](int rk, float wk) {
    const bool ok = rk >= 0;
    const float4* src = reinterpret_cast<const float4*>(r.rec_out + ((ok ? rk : 0) * rec_rows + hrow) * kD) + 2 * c;
    const float4 v0 = src[0];
    const float4 v1 = src[1];
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, ok ? x[e] : 0.f, acc[e]);
  };
  const int n0 = n < kWaveSize ? n : kWaveSize;
#pragma unroll 4
  for (int k0 = 0; k0 < n0; k0 += kMergeGroups) {
    const int k = k0 + grp;  // below 64; lanes at or past n hold record -1
    fold(__shfl(rc0, k), __shfl(w0, k));
  }
  for (int k0 = kWaveSize; k0 < n; k0 += kMergeGroups) {
    const int k = k0 + grp;
    const int rk = k < n ? rec_of(k) : -1;
    fold(rk, rk < 0 ? 0.f : expf(lse_of(rk) - ms));
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
template <class C>
constexpr bool two_waves_per_simd() {
  return std::is_same<C, MfmaFP4>::value;
}

template <class C, int G>
hipError_t launch_group(const DecodeArgs& a, const RowsArgs& r, hipStream_t s) {
  if (r.head_group == 8) {
    if constexpr (two_waves_per_simd<C>())
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, 2 * kDecodeThreads>), dim3(r.num_wg),
                         dim3(2 * kDecodeThreads), 0, s, a, r);
    else
      hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 2, kDecodeThreads>), dim3(r.num_wg), dim3(kDecodeThreads),
                         0, s, a, r);
  } else
    hipLaunchKernelGGL((paged_decode_rows_kernel<C, G, 1, kDecodeThreads>), dim3(r.num_wg), dim3(kDecodeThreads), 0,
                       s, a, r);
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
  return decode_mfma_supported(act, cache, head_dim, group, block_size) && num_kv_heads % 4 == 0;
}

hipError_t launch_paged_decode_rows(const DecodeArgs& a, const RowsArgs& r, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, r, G, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, r, G, s);
  if (cache == LGM_FP4_E2M1) return dispatch<MfmaFP4>(a, r, G, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
