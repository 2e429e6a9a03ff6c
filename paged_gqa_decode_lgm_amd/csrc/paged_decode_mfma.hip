// Split-K paged GQA decode attention with matrix cores, for gfx950: bf16 or
// FP8 E4M3 caches, head_dim 128, block_size 16, group size G <= 16.
//
// The method is the one of paged_decode.hip (mainarch README, decode-attention
// section; Loom Kernels README, "Attention" row): partitions of the context
// processed independently with an online softmax, merged by log-sum-exp, each
// KV row read once for its G query heads.  Two things change on this chip.
//
// Arithmetic: with G query heads sharing a KV head, the scores of a 16-token
// block and the probability-weighted sum of V rows are small dense
// contractions, so both go to v_mfma_f32_16x16x32_bf16 and the vector ALU only
// runs the softmax bookkeeping (operand layouts and the per-tile update are in
// mfma_common.h).  The probabilities enter the MFMA rounded to bf16 and the
// output is normalised by the sum of those same rounded values, so it is an
// exact convex combination of V rows up to fp32 accumulation; the log-sum-exp
// uses the unrounded sum.
//
// Scheduling: a grid of one workgroup per (partition, kv head, sequence)
// dispatches in order, so with ragged batches the empty partitions of short
// sequences sit between live ones and hold up dispatch, and the workgroups
// that land on one XCD are fixed in advance even though XCDs do not stream
// all kv heads at the same speed.  Instead a persistent grid (the resident
// capacity of the chip) pulls work items from an atomic counter.  The items
// are the live (sequence, partition, kv head) triples only, the full-size
// partitions first and the shorter tail partitions last; every workgroup
// walks the context lengths 64 sequences at a time with a wave prefix sum to
// turn an item number into its triple.
#include <mutex>

#include "mfma_common.h"

namespace lgm {
namespace {

using namespace mfma;

// Item number -> (sequence, partition, kv head).  First come the full
// partitions of every sequence (phase 0), then the shorter tail partitions
// that cover the rest of each context (phase 1), so the queue drains on short
// items.  Within a phase the items of sequence b are consecutive numbers,
// partition-major, kv head fastest (the kv heads of one partition read the
// same blocks at about the same time).  Wave 0 walks the context lengths 64
// sequences at a time with a wave prefix sum; the walk only moves forward (a
// workgroup's item numbers increase) and its state stays in LDS between
// items, so none of it occupies registers during the tile loop.
struct CursorSmem {
  int incl[kWaveSize];  // inclusive item counts of the chunk's sequences
  int ctx[kWaveSize];   // their clamped context lengths
  int phase, base_b, base_item, total;
};
struct ItemSlot {
  int b, part, g, ctx;  // b < 0: no item left
};

// Loads the chunk of sequences base_b .. base_b + 63 for `phase`; returns its item count.
__device__ __forceinline__ int cursor_load(const DecodeArgs& p, CursorSmem& cs, int phase, int base_b, int lane) {
  const int bb = base_b + lane;
  int c = 0, items = 0;
  if (bb < p.dims.num_seqs) {
    c = p.context_lens[bb];
    c = c < 0 ? 0 : (c > p.max_context_len ? p.max_context_len : c);
    const int nfull = p.parts.nfull(c);
    items = (phase == 0 ? nfull : p.parts.count(c) - nfull) * p.dims.num_kv_heads;
  }
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) {
    const int t = __shfl_up(items, o);
    if (lane >= o) items += t;
  }
  cs.incl[lane] = items;
  cs.ctx[lane] = c;
  return __builtin_amdgcn_readlane(items, kWaveSize - 1);
}

// Wave 0 only: the triple of `item` into `out`.
__device__ __forceinline__ void cursor_locate(const DecodeArgs& p, CursorSmem& cs, int item, int lane,
                                              ItemSlot& out) {
  int phase = __builtin_amdgcn_readfirstlane(cs.phase);
  int base_b = __builtin_amdgcn_readfirstlane(cs.base_b);
  int base_item = __builtin_amdgcn_readfirstlane(cs.base_item);
  int total = __builtin_amdgcn_readfirstlane(cs.total);
  bool found = item >= 0;  // a negative item (counters not zero on entry) is no item
  while (found && item >= base_item + total) {
    base_item += total;
    if (base_b + kWaveSize < p.dims.num_seqs) {
      base_b += kWaveSize;
    } else if (phase == 0) {
      phase = 1;
      base_b = 0;
    } else {
      total = 0;
      found = false;
      break;
    }
    total = cursor_load(p, cs, phase, base_b, lane);
  }
  int b = -1, part = 0, g = 0, ctx = 0;
  if (found) {
    const uint64_t above = __ballot(base_item + cs.incl[lane] > item);
    const int j = __builtin_ctzll(above);
    const int excl = j == 0 ? 0 : cs.incl[j - 1];
    const int r = item - base_item - excl;
    const int within = r / p.dims.num_kv_heads;
    g = r - within * p.dims.num_kv_heads;
    b = base_b + j;
    ctx = cs.ctx[j];
    part = phase == 0 ? within : p.parts.nfull(ctx) + within;
  }
  if (lane == 0) {
    cs.phase = phase;
    cs.base_b = base_b;
    cs.base_item = base_item;
    cs.total = total;
    out.b = b;
    out.part = part;
    out.g = g;
    out.ctx = ctx;
  }
}

template <int G>
struct DecodeSmem {
  // Wave states of an item, double-buffered by item parity: the next item's
  // waves write one buffer while the other still holds this item's states.
  float acc[2][kNW][G][kD];
  float m[2][kNW][G];
  float l[2][kNW][G];   // sums of the bf16-rounded probabilities (normalise the output)
  float le[2][kNW][G];  // sums of the fp32 probabilities (the log-sum-exp)
  ItemSlot slot[2];     // the current and the next item, by item parity
  CursorSmem cursor;
};

// One item's values, uniform across the workgroup.
struct Item {
  int b, g, part, nparts, start, end, nsteps;
};

template <class C>
__device__ __forceinline__ Item read_item(const DecodeArgs& p, const ItemSlot& sl) {
  constexpr int kStepTokens = step_blocks<C>() * kBS;
  Item it;
  it.b = __builtin_amdgcn_readfirstlane(sl.b);
  it.g = __builtin_amdgcn_readfirstlane(sl.g);
  it.part = __builtin_amdgcn_readfirstlane(sl.part);
  const int ctx = __builtin_amdgcn_readfirstlane(sl.ctx);
  it.nparts = p.parts.count(ctx);
  p.parts.range(ctx, it.part, it.start, it.end);
  it.nsteps = (it.end - it.start + kStepTokens - 1) / kStepTokens;
  return it;
}

// Steps of the item this wave takes: wave, wave + 4, ...
__device__ __forceinline__ int wave_steps(const Item& it, int wave) {
  return it.nsteps > wave ? (it.nsteps - wave + kNW - 1) / kNW : 0;
}

// Block ids of this wave's steps k0 .. k0 + 64/NB - 1 of the item, one per
// lane (lane NB*k + h holds block h of the wave's step k0 + k), read back
// with readlane so no table load sits between a step and its K/V loads.  -1
// marks an absent block (past the end) or an out-of-range table entry.
template <int NB>
__device__ __forceinline__ int preload_ids(const DecodeArgs& p, const Item& it, int k0, int lane, int wave) {
  const int MB = p.dims.max_blocks_per_seq;
  const __amdgpu_buffer_rsrc_t bt_rs = span_rsrc(p.block_tables + (int64_t)it.b * MB, MB * 4);
  const int t = wave + kNW * (k0 + lane / NB);
  const int lb = it.start / kBS + NB * t + lane % NB;
  const int lb_end = (it.end + kBS - 1) / kBS;
  const int id = buf_load4(bt_rs, 4 * (lb < MB ? lb : 0));
  return (t < it.nsteps && lb < lb_end && (unsigned)id < (unsigned)p.dims.num_blocks) ? id : -1;
}

// Starts an item for this wave: the query operand (with the score scale's
// sign folded in; the positive scale is returned), the block ids of its first
// steps and the K/V loads of its first step are issued here, so that they are
// in flight while the previous item is merged and stored.
template <class C, int G>
__device__ __forceinline__ float begin_item(const DecodeArgs& p, const Item& it, int lane, int wave, short8 (&qb)[4],
                                            int& ids, int (&pid)[step_blocks<C>()],
                                            StepRegs<C, step_blocks<C>()>& sr) {
  constexpr int NB = step_blocks<C>();
  const bool qvec = ((uintptr_t)p.q % 16 == 0) && (p.q_seq_stride % 8 == 0);
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)it.b * p.q_seq_stride + (int64_t)it.g * G * kD;
  load_q_operand<C, G>(qb, qrow, qvec, lane & 15, lane >> 4);
  float c = p.softmax_scale * kLog2e;
  if constexpr (C::kFp8) c *= kv_scale(p.k_scale, p.flags, it.g);
  const float csc = fold_score_scale(c, qb);
  if (wave_steps(it, wave) > 0) {
    ids = preload_ids<NB>(p, it, 0, lane, wave);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) pid[bb] = __builtin_amdgcn_readlane(ids, bb);
    load_step_k<C, NB>(p, it.g, pid, lane, sr);
    __builtin_amdgcn_sched_barrier(0);  // K before V, as inside the step loop
    load_step_v<C, NB>(p, it.g, pid, lane, sr);
  }
  return csc;
}

// The wave's steps of an item into st.  One register set per operand: the
// next step's K loads are issued as soon as the score MFMAs have consumed the
// current K, and its V loads as soon as the output MFMAs have consumed the
// current V, so loads stay in flight through all of a step's arithmetic.
// Wave 0's lane 0 claims the workgroup's next item two steps before the end
// (into `next`): late enough that items are claimed in about the order they
// start, early enough that the claim is back before the merge needs it.
template <class C, int G>
__device__ __forceinline__ void run_steps(const DecodeArgs& p, const Item& it, int lane, int wave,
                                          const short8 (&qb)[4], float csc, int ids, int (&pid)[step_blocks<C>()],
                                          StepRegs<C, step_blocks<C>()>& sr, WaveState& st, int& next) {
  constexpr int NB = step_blocks<C>();
  constexpr int SPW = kWaveSize / NB;  // steps per window of block ids
  const int my_steps = wave_steps(it, wave);
  const int claim_at = my_steps > 2 ? my_steps - 2 : 0;
  const bool claimer = wave == 0;
  if (claimer && my_steps == 0 && lane == 0) next = (int)gridDim.x + atomicAdd(p.work_counters, 1);
  for (int k = 0; k < my_steps; ++k) {
    if (claimer && k == claim_at && lane == 0) next = (int)gridDim.x + atomicAdd(p.work_counters, 1);
    const int t = wave + kNW * k;
    float4v s[NB];
    step_scores<C, NB>(sr, qb, s);
    // Next step's K.  After the last step the blocks are absent, so every
    // iteration issues the same loads in the same order and the compiler can
    // wait for K alone.
    int nid[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) nid[bb] = -1;
    if (k + 1 < my_steps) {
      if (((k + 1) % SPW) == 0) ids = preload_ids<NB>(p, it, k + 1, lane, wave);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) nid[bb] = __builtin_amdgcn_readlane(ids, NB * ((k + 1) % SPW) + bb);
    }
    load_step_k<C, NB>(p, it.g, nid, lane, sr);
    uint32_t valid = 0;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) valid |= (pid[bb] >= 0 ? 1u : 0u) << bb;
    step_update<C, NB>(st, sr, s, csc, valid, it.start + NB * kBS * t, it.end, lane >> 4);
    load_step_v<C, NB>(p, it.g, nid, lane, sr);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) pid[bb] = nid[bb];
  }
}

// Wave epilogue: complete the denominators and publish this wave's state.
// The rounded-probability sum of head 4kg + j sits in psum[j] of lane group
// kg; the reference and the fp32 sum of head n in lane n.
template <int G>
__device__ __forceinline__ void publish_state(DecodeSmem<G>& sm, int buf, const WaveState& st, int lane, int wave) {
  const int n = lane & 15, kg = lane >> 4;
  const float lsum_e = sum4(st.lsum_e);
  if (kg == 0 && n < G) {
    sm.m[buf][wave][n] = st.m;
    sm.le[buf][wave][n] = lsum_e;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * kg + j;
    if (h < G) {
      if (n == 0) sm.l[buf][wave][h] = st.psum[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.acc[buf][wave][h][8 * n + i] = st.acc[i][j];
    }
  }
}

// Merges the four wave states of an item and writes the final output (one
// partition) or the partition's record.
template <class C, int G>
__device__ __forceinline__ void merge_and_store(const DecodeArgs& p, const DecodeSmem<G>& sm, int buf, const Item& it,
                                                int tid) {
  const float vscale = C::kFp8 ? kv_scale(p.v_scale, p.flags, it.g) : 1.f;
  for (int idx = tid; idx < G * kD; idx += kDecodeThreads) {
    const int h = idx / kD;
    const int d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm.m[buf][w][h]);
    const float ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, Le = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = fast_exp2(sm.m[buf][w][h] - ms);
      L += sm.l[buf][w][h] * f;
      Le += sm.le[buf][w][h] * f;
      o += sm.acc[buf][w][h][d] * f;
    }
    o = L > 0.f ? o / L : 0.f;
    o *= vscale;
    const float lse = Le > 0.f ? (ms + fast_log2(Le)) * kLn2 : -INFINITY;
    const int64_t row = (int64_t)it.b * p.dims.num_q_heads + it.g * G + h;
    if (it.nparts == 1) {
      static_cast<uint16_t*>(p.out)[row * kD + d] = f32_to_bf16_rne(o);
      if (d == 0 && p.out_lse) p.out_lse[row] = lse;
    } else {
      p.part_out[(row * p.max_partitions + it.part) * kD + d] = o;
      if (d == 0) p.part_lse[row * p.max_partitions + it.part] = lse;
    }
  }
}

// Persistent workgroup: items blockIdx.x, then gridDim.x + (counter value) for
// every further item.  Per item the four waves run their tiles, publish their
// states and meet at one barrier, behind which wave 0 has placed the next
// item; each wave then starts the next item's loads before merging and
// storing this one.  counters[0] hands out items, counters[1] counts
// workgroups that have run out of items; the last one to run out puts both
// back to zero, so the next launch finds them zero.  A workgroup increments
// counters[1] only after its final fetch from counters[0] has returned (its
// exit depends on the fetched value), so no fetch follows the reset.
template <class C, int G>
__global__ __launch_bounds__(kDecodeThreads, 2) void paged_decode_mfma_kernel(DecodeArgs p) {
  static_assert(G >= 1 && G <= 16, "group size");
  __shared__ DecodeSmem<G> sm;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  int32_t* counters = p.work_counters;

  if (wave == 0) {
    const int total = cursor_load(p, sm.cursor, 0, 0, lane);
    if (lane == 0) {
      sm.cursor.phase = 0;
      sm.cursor.base_b = 0;
      sm.cursor.base_item = 0;
      sm.cursor.total = total;
    }
    cursor_locate(p, sm.cursor, blockIdx.x, lane, sm.slot[0]);
  }
  __syncthreads();
  constexpr int NB = step_blocks<C>();
  Item it = read_item<C>(p, sm.slot[0]);
  short8 qb[4];
  StepRegs<C, NB> sr;
  int ids = 0, pid[NB];
  float csc = 1.f;
  if (it.b >= 0) csc = begin_item<C, G>(p, it, lane, wave, qb, ids, pid, sr);
  for (int k = 0; it.b >= 0; ++k) {
    // Lane-derived addresses are loop-invariant; recomputing them per item
    // (instead of keeping them live across every step) keeps the step loop
    // within its register budget.
    int lane_i = lane, tid_i = threadIdx.x;
    asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    WaveState st;
    st.reset();
    int next = 0;
    run_steps<C, G>(p, it, lane_i, wave, qb, csc, ids, pid, sr, st, next);
    publish_state<G>(sm, k & 1, st, lane_i, wave);
    if (wave == 0) cursor_locate(p, sm.cursor, __builtin_amdgcn_readlane(next, 0), lane_i, sm.slot[(k + 1) & 1]);
    __syncthreads();
    const Item nx = read_item<C>(p, sm.slot[(k + 1) & 1]);
    if (nx.b >= 0) csc = begin_item<C, G>(p, nx, lane_i, wave, qb, ids, pid, sr);
    merge_and_store<C, G>(p, sm, k & 1, it, tid_i);
    it = nx;
  }
  if (threadIdx.x == 0 && atomicAdd(counters + 1, 1) == (int)gridDim.x - 1) {
    atomicExch(counters, 0);
    atomicExch(counters + 1, 0);
  }
}

// Resident workgroups per compute unit of each instantiation, queried once.
template <class C, int G>
int resident_per_cu() {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, paged_decode_mfma_kernel<C, G>, kDecodeThreads, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  return occ;
}

template <class C, int G>
hipError_t launch_persistent(const DecodeArgs& a, int compute_units, hipStream_t s) {
  const int64_t per_cu = resident_per_cu<C, G>();
  const int64_t upper = (int64_t)a.dims.num_seqs * a.dims.num_kv_heads * a.max_partitions;
  int64_t grid = compute_units * (per_cu < kPersistentMaxPerCU ? per_cu : kPersistentMaxPerCU);
  if (grid > upper) grid = upper;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((paged_decode_mfma_kernel<C, G>), dim3((unsigned)grid), dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

template <class C>
hipError_t dispatch(const DecodeArgs& a, int G, int compute_units, hipStream_t s) {
  switch (G) {
#define LGM_CASE(GV) \
  case GV:           \
    return launch_persistent<C, GV>(a, compute_units, s);
    LGM_CASE(1) LGM_CASE(2) LGM_CASE(3) LGM_CASE(4) LGM_CASE(5) LGM_CASE(6) LGM_CASE(7) LGM_CASE(8)
    LGM_CASE(9) LGM_CASE(10) LGM_CASE(11) LGM_CASE(12) LGM_CASE(13) LGM_CASE(14) LGM_CASE(15) LGM_CASE(16)
#undef LGM_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// Compute units of the device a stream runs on, queried once per device
// (std::call_once, so threads making their first calls together agree).
int compute_units_of(hipStream_t s) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static int cache[kMaxDevices];
  int dev = 0;
  if (s == nullptr || hipStreamGetDevice(s, &dev) != hipSuccess) {
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  }
  if (dev < 0 || dev >= kMaxDevices) dev = 0;
  std::call_once(once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    cache[dev] = n;
  });
  return cache[dev];
}

}  // namespace

bool decode_mfma_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size) {
  return act == LGM_BF16 && (cache == LGM_BF16 || cache == LGM_FP8_E4M3 || cache == LGM_FP4_E2M1) &&
         head_dim == kD && group >= 1 && group <= 16 && block_size == kBS;
}

hipError_t launch_paged_decode_mfma(const DecodeArgs& a, lgm_dtype cache, hipStream_t s) {
  const int G = a.dims.num_q_heads / a.dims.num_kv_heads;
  const int cus = compute_units_of(s);
  if (cache == LGM_BF16) return dispatch<MfmaBF16>(a, G, cus, s);
  if (cache == LGM_FP8_E4M3) return dispatch<MfmaFP8>(a, G, cus, s);
  if (cache == LGM_FP4_E2M1) return dispatch<MfmaFP4>(a, G, cus, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
