// C-ABI host layer: validates every host-visible argument before any HIP
// call, resolves the partition plan, and launches the kernels on the
// caller's stream.  A call either meets its full contract or returns an
// error and does nothing (Loom Kernels README, «Architecture»); error text
// names the function, the
// argument and what was expected (the span check of mainarch's VA guard,
// troubleshooting section, is the model).  Nothing here allocates device or
// host memory.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>
#include <string>

#include "lgm_internal.h"
#include "lgm_mla.h"
#include "lgm_probe.h"

namespace {

thread_local std::string g_err;

lgm_status fail(lgm_status st, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = std::string(fn) + ": " + buf;
  return st;
}

const char* dtype_name(lgm_dtype t) {
  switch (t) {
    case LGM_F32: return "LGM_F32";
    case LGM_BF16: return "LGM_BF16";
    case LGM_FP8_E4M3: return "LGM_FP8_E4M3";
    case LGM_FP4_E2M1: return "LGM_FP4_E2M1";
  }
  return "invalid";
}

bool dtype_valid(int t) { return t == LGM_F32 || t == LGM_BF16 || t == LGM_FP8_E4M3 || t == LGM_FP4_E2M1; }

int64_t elem_bytes(lgm_dtype t) { return t == LGM_F32 ? 4 : (t == LGM_BF16 ? 2 : 1); }

struct Span {
  const char* name;
  uintptr_t lo;
  int64_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.lo || !b.lo || a.bytes <= 0 || b.bytes <= 0) return false;
  return a.lo < b.lo + (uintptr_t)b.bytes && b.lo < a.lo + (uintptr_t)a.bytes;
}

// Shared dims checks.  head_dim / block_size support is checked by the caller.
lgm_status check_dims(const char* fn, const lgm_paged_dims& d) {
  if (d.num_seqs < 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_seqs = %d must be >= 0", d.num_seqs);
  if (d.num_q_heads < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_q_heads = %d must be >= 1", d.num_q_heads);
  if (d.num_kv_heads < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_kv_heads = %d must be >= 1", d.num_kv_heads);
  if (d.num_q_heads % d.num_kv_heads != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_q_heads = %d must be a multiple of dims.num_kv_heads = %d",
                d.num_q_heads, d.num_kv_heads);
  if (d.head_dim < 2 || d.head_dim % 2 != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.head_dim = %d must be even and >= 2", d.head_dim);
  if (d.block_size < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.block_size = %d must be >= 1", d.block_size);
  if (d.num_blocks < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_blocks = %d must be >= 1", d.num_blocks);
  if (d.max_blocks_per_seq < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.max_blocks_per_seq = %d must be >= 1", d.max_blocks_per_seq);
  if ((int64_t)d.max_blocks_per_seq * d.block_size > INT32_MAX)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.max_blocks_per_seq * dims.block_size = %lld exceeds INT32_MAX",
                (long long)d.max_blocks_per_seq * d.block_size);
  return LGM_OK;
}

// Bytes of one cache pool.  FP4 blocks hold their codes (D/2 bytes per
// token and kv head) and then their E8M0 scales (D/32 bytes).
int64_t cache_bytes(const lgm_paged_dims& d, lgm_dtype cache) {
  const int64_t rows = (int64_t)d.num_blocks * d.block_size * d.num_kv_heads;
  if (cache == LGM_FP4_E2M1) return rows * (d.head_dim / 2 + d.head_dim / 32);
  return rows * d.head_dim * elem_bytes(cache);
}

lgm_status check_scales(const char* fn, lgm_dtype cache, const float* k_scale, const float* v_scale) {
  if (cache == LGM_FP8_E4M3) {
    if (!k_scale) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "k_scale is NULL; LGM_FP8_E4M3 caches need fp32 [num_kv_heads] scales");
    if (!v_scale) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "v_scale is NULL; LGM_FP8_E4M3 caches need fp32 [num_kv_heads] scales");
  } else {
    if (k_scale || v_scale)
      return fail(LGM_ERR_INVALID_ARGUMENT, fn, "k_scale / v_scale must be NULL for a %s cache", dtype_name(cache));
  }
  return LGM_OK;
}

// Contract-variant flags: only the bits a call documents, and the per-tensor
// scale only for FP8 caches.
lgm_status check_flags(const char* fn, uint32_t flags, uint32_t allowed, lgm_dtype cache) {
  if (flags & ~allowed)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "flags = 0x%x: only 0x%x (%s) are defined for this call", flags,
                allowed, allowed & LGM_ROPE_INTERLEAVED
                             ? "LGM_ROPE_INTERLEAVED | LGM_CACHE_HND | LGM_SCALE_PER_TENSOR"
                             : "LGM_CACHE_HND | LGM_SCALE_PER_TENSOR");
  if ((flags & LGM_SCALE_PER_TENSOR) && cache != LGM_FP8_E4M3)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "flags: LGM_SCALE_PER_TENSOR needs an LGM_FP8_E4M3 cache, not %s",
                dtype_name(cache));
  return LGM_OK;
}

// Bytes of the k_scale / v_scale arrays a call reads.
int64_t scale_bytes(const float* s, const lgm_paged_dims& d, uint32_t flags) {
  return s ? ((flags & LGM_SCALE_PER_TENSOR) ? 4 : (int64_t)d.num_kv_heads * 4) : 0;
}

lgm_status check_no_alias(const char* fn, const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(LGM_ERR_INVALID_ARGUMENT, fn, "output '%s' overlaps output '%s'", outs[i].name, outs[j].name);
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(LGM_ERR_INVALID_ARGUMENT, fn, "output '%s' overlaps input '%s' (%lld bytes at %p)", outs[i].name,
                    ins[j].name, (long long)ins[j].bytes, (void*)ins[j].lo);
  }
  return LGM_OK;
}

constexpr int kAutoTargetWorkgroups = 8192;
#ifndef LGM_TAIL_DIVISOR
#define LGM_TAIL_DIVISOR 2
#endif
constexpr int kTailDivisor = LGM_TAIL_DIVISOR;
constexpr int kMinAutoPartitionBlocks = 4;

// Partition plan: returns the partition size in tokens, or -1 after setting the error.
// (partition_size 0 reaches here only for the vector-ALU shapes: the
// matrix-core shapes take the single-launch or whole-row plan.)
int32_t resolve_partition(const char* fn, const lgm_paged_dims& d, int32_t max_ctx, int32_t ps) {
  if (ps < 0) {
    fail(LGM_ERR_INVALID_ARGUMENT, fn, "partition_size = %d must be 0 (library chooses) or positive", ps);
    return -1;
  }
  if (ps > 0 && ps % d.block_size != 0) {
    fail(LGM_ERR_INVALID_ARGUMENT, fn, "partition_size = %d must be a multiple of dims.block_size = %d", ps,
         d.block_size);
    return -1;
  }
  const int64_t cap = ((int64_t)(max_ctx > 0 ? max_ctx : 1) + d.block_size - 1) / d.block_size * d.block_size;
  if (ps == 0) {
    // Enough partitions that the grid holds ~kAutoTargetWorkgroups workgroups
    // at the longest context, but never fewer than 4 blocks (one per wave).
    const int64_t units = (int64_t)(d.num_seqs > 0 ? d.num_seqs : 1) * d.num_kv_heads;
    const int64_t parts = (kAutoTargetWorkgroups + units - 1) / units;
    int64_t p = (cap + parts - 1) / parts;
    const int64_t step = 2 * (int64_t)d.block_size;  // whole 32-token tiles of the decode kernels
    p = (p + step - 1) / step * step;
    const int64_t minp = (int64_t)kMinAutoPartitionBlocks * d.block_size;
    ps = (int32_t)(p < minp ? minp : p);
  }
  return (int32_t)(ps < cap ? ps : cap);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr size_t kCounterSlot = LGM_COUNTER_SLOT_BYTES;  // the counters at the start of every workspace

// kv heads per whole-row workgroup: 8 (whole NHD rows) when they divide the
// kv heads and the group has at most 8 query heads per kv head, else 4, else
// (2 or 1, whole rows of 2 or 1 kv heads) as many as divide the kv heads,
// each head's tiles then dealt to 2 or 4 waves in token slices.  A
// segment's staged query rows and results grow with G (128 rows of 272 +
// 512 bytes at G = 16 and 8 heads), and past 8 a batch holds a single
// segment, so a range's second segment waits for the first one's flush and
// restarts the load pipeline.  Call medians at G = 16 (8 kv heads, 4 vs 8
// heads per workgroup): bf16 200 vs 206 us (64 contexts of 512..8192), FP8
// 139-141 vs 147 us (128 of 1024..4096); at G = 8 FP8 was 1.5% slower with 4.
static int rows_head_group(int num_kv_heads, int G) {
  if (num_kv_heads % 8 == 0 && G <= LGM_ROWS_HG8_MAX_GROUP) return 8;
  if (num_kv_heads % 4 == 0) return 4;
  return num_kv_heads % 2 == 0 ? 2 : 1;
}

// Launch plan of one attention call, a function of host-visible arguments only.
// Every plan that needs a workspace lays it out the same way at the start:
// the counter slot (LGM_COUNTER_SLOT_BYTES): the work-queue kernel's two
// counters, then the single-launch kernel's arrival counters, one per
// (sequence, kv head) stream.  Each kernel leaves the counters it uses zero,
// and no plan puts anything else there, so one zero-filled workspace may
// serve calls on any plan in turn.  The plan's own regions follow.
struct Plan {
  bool fused;       // single-launch split kernel (small jobs): partitions of ps tokens, merged in the launch
  bool rows;        // whole-row kernel: equal tile ranges (partition_size 0) ...
  bool rows_parts;  // ... or equal runs of whole partitions (an explicit partition_size of whole tiles; an
                    // even Hkv: four slices of one head's partition held up the 1-kv-head shape, 60 vs 54 us)
  lgm::PartitionPlan parts;
  int32_t ps, P;
  size_t counters_bytes, part_out_bytes, part_lse_bytes;
  int32_t W, HG;  // rows: workgroups (ranges), kv heads per workgroup
  int32_t chunk_steps, nchunks;  // fused: 32-token steps per wave per partition, partitions per context
  size_t rec_out_bytes, rec_lse_bytes, stream_bytes;
  size_t total;
};

// Whole-row plan: one range per compute unit of MI355X (256 CUs, one
// workgroup each, so no range runs beside another that the CU favours),
// fewer for small batches so that a range holds at least kRowsMinTiles tiles.
#ifndef LGM_ROWS_WORKGROUPS
#define LGM_ROWS_WORKGROUPS 256
#endif
constexpr int64_t kRowsWorkgroups = LGM_ROWS_WORKGROUPS;
#ifndef LGM_ROWS_MIN_TILES
#define LGM_ROWS_MIN_TILES 2
#endif
constexpr int64_t kRowsMinTiles = LGM_ROWS_MIN_TILES;
constexpr int64_t kRowsTile = 32;
// Whole-row partition plan: explicit partition sizes of at least this many
// tokens (and whole 32-token tiles), when the longest context holds at least
// kRowsMinPartitions of them and the batch at least one unit per range.  The
// ranges hold whole partitions in equal numbers, which balances long
// contexts; with only a few partitions per range, ragged contexts leave the
// ranges unequal by up to a partition, and the work-queue kernel is faster
// (measured: 131072-token contexts, partitions of 512: 386 vs 406 us; 64
// contexts of 512..8192 tokens, partitions of 512: 263 vs 239 us).
#ifndef LGM_ROWS_MIN_PARTITION
#define LGM_ROWS_MIN_PARTITION 256
#endif
constexpr int32_t kRowsMinPartition = LGM_ROWS_MIN_PARTITION;
constexpr int32_t kRowsMinPartitions = 64;

// Single-launch split plan: taken with partition_size 0 on the matrix-core
// shapes when the job is small or middling: at most kFusedMaxStreams
// (sequence, kv head) streams and at most kFusedMaxTiles 32-token tiles over
// them at max_context_len (twice that for FP8 caches, whose tiles are half
// the bytes).  Measured on MI355X (uniform contexts, partition_size 0, call
// times): the whole-row and work-queue plans pay a fixed cost that dominates
// such jobs (8 x 8 kv heads x 2048 tokens: 15.5 us single launch against 26.5
// us whole-row; 128 x 2 x 2048: 41.8 against 57.0 us work queue), while from
// about 28672 bf16 tiles the whole-row plan streams faster (7 x 8 x 16384:
// 86 against 93 us; 32 x 8 x 8192: 172 against 192 us; FP8 64 x 8 x 4096:
// 99 against 109 us).
#ifndef LGM_FUSED_MAX_TILES
#define LGM_FUSED_MAX_TILES 16384
#endif
constexpr int64_t kFusedMaxTiles = LGM_FUSED_MAX_TILES;
#ifndef LGM_FUSED_TARGET_WORKGROUPS
#define LGM_FUSED_TARGET_WORKGROUPS 256
#endif
constexpr int64_t kFusedTargetWorkgroups = LGM_FUSED_TARGET_WORKGROUPS;
constexpr int64_t kFusedPartStep = 128;
constexpr int64_t kFusedMaxSteps = 32;  // 32-token steps per wave in one partition
#ifndef LGM_FUSED_WG_OVERHEAD
#define LGM_FUSED_WG_OVERHEAD 128
#endif
constexpr int64_t kFusedWorkgroupOverhead = LGM_FUSED_WG_OVERHEAD;  // tokens' worth of fixed latency per workgroup

// Partition of the single-launch plan: over 1..kFusedMaxChunks partitions per
// context (whole 128-token steps, at most kFusedMaxSteps per wave), the one
// whose slowest compute unit has the least to read when the
// streams * partitions workgroups are spread kFusedTargetWorkgroups at a
// time: rounds * partition tokens.  Ties go to fewer partitions (fewer
// records to merge).  0 if no partition fits.
int64_t fused_partition(int64_t streams, int64_t max_ctx) {
  int64_t best = 0, best_cost = 0;
  for (int64_t n = 1; n <= lgm::kFusedMaxChunks; ++n) {
    int64_t part = (max_ctx + n - 1) / n;
    part = (part + kFusedPartStep - 1) / kFusedPartStep * kFusedPartStep;
    part = part < kFusedPartStep ? kFusedPartStep : part;
    if (part / kFusedPartStep > kFusedMaxSteps) continue;
    const int64_t used = (max_ctx + part - 1) / part;
    const int64_t rounds = (streams * (used < 1 ? 1 : used) + kFusedTargetWorkgroups - 1) / kFusedTargetWorkgroups;
    const int64_t cost = rounds * (part + kFusedWorkgroupOverhead);
    if (best == 0 || cost < best_cost) {
      best = part;
      best_cost = cost;
    }
  }
  return best;
}

lgm_status plan_decode(const char* fn, const lgm_paged_dims& d, int32_t max_ctx, int32_t ps_arg, lgm_dtype cache,
                       Plan& pl) {
  pl = Plan{};
  const int G = d.num_q_heads / d.num_kv_heads;
  const lgm_dtype act = cache == LGM_F32 ? LGM_F32 : LGM_BF16;  // the only supported pairings
  const bool persistent = lgm::decode_mfma_supported(act, cache, d.head_dim, G, d.block_size);
  if (ps_arg == 0 && persistent) {
    const int64_t streams = (int64_t)d.num_seqs * d.num_kv_heads;
    const int64_t tiles = streams * (((int64_t)max_ctx + kRowsTile - 1) / kRowsTile);
    const int64_t max_tiles = cache == LGM_FP8_E4M3 ? 2 * kFusedMaxTiles : kFusedMaxTiles;
    const int64_t part = streams <= lgm::kFusedMaxStreams && tiles <= max_tiles ? fused_partition(streams, max_ctx) : 0;
    if (part > 0) {
      pl.fused = true;
      pl.ps = (int32_t)part;
      pl.chunk_steps = (int32_t)(part / kFusedPartStep);
      pl.nchunks = (int32_t)(((int64_t)max_ctx + part - 1) / part);
      pl.nchunks = pl.nchunks < 1 ? 1 : pl.nchunks;
      pl.P = pl.nchunks;
      pl.counters_bytes = kCounterSlot;
      if (pl.nchunks > 1) {
        pl.rec_out_bytes = align256((size_t)streams * pl.nchunks * G * d.head_dim * sizeof(float));
        pl.rec_lse_bytes = align256((size_t)streams * pl.nchunks * G * sizeof(float));
      }
      pl.total = pl.counters_bytes + pl.rec_out_bytes + pl.rec_lse_bytes;
      return LGM_OK;
    }
  }
  if (ps_arg == 0 && lgm::decode_rows_supported(act, cache, d.head_dim, d.num_kv_heads, G, d.block_size)) {
    pl.rows = true;
    pl.HG = rows_head_group(d.num_kv_heads, G);
    const int64_t streams = (int64_t)d.num_seqs * (d.num_kv_heads / pl.HG);
    const int64_t tiles = streams * ((max_ctx + kRowsTile - 1) / kRowsTile);
    // The kernel cuts its ranges in cost units: 4 per tile and at most 16 * 8 / HG per stream.
    if (4 * tiles + 128 * streams > (int64_t)INT32_MAX)
      return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs * head groups * tiles = %lld: too many", (long long)tiles);
    if ((int64_t)d.num_seqs * d.num_q_heads > (int64_t)INT32_MAX - 1024)  // merge rows are int-indexed
      return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs * num_q_heads = %lld: too many",
                  (long long)d.num_seqs * d.num_q_heads);
    int64_t W = (tiles + kRowsMinTiles - 1) / kRowsMinTiles;
    W = W < 1 ? 1 : (W > kRowsWorkgroups ? kRowsWorkgroups : W);
    pl.W = (int32_t)W;
    const size_t rows_per_rec = (size_t)pl.HG * G;
    pl.counters_bytes = kCounterSlot;
    pl.rec_out_bytes = align256((size_t)W * 2 * rows_per_rec * d.head_dim * sizeof(float));
    pl.rec_lse_bytes = align256((size_t)W * 2 * rows_per_rec * sizeof(float));
    pl.stream_bytes = align256((size_t)streams * sizeof(int32_t));
    pl.total = pl.counters_bytes + pl.rec_out_bytes + pl.rec_lse_bytes + 2 * pl.stream_bytes;
    return LGM_OK;
  }
  pl.ps = resolve_partition(fn, d, max_ctx, ps_arg);
  if (pl.ps < 0) return LGM_ERR_INVALID_ARGUMENT;
  const int32_t most_parts = (int32_t)(((int64_t)max_ctx + pl.ps - 1) / pl.ps);
  const int64_t est_units = (int64_t)d.num_seqs * (d.num_kv_heads / rows_head_group(d.num_kv_heads, G)) * most_parts;
  if (ps_arg > 0 && pl.ps >= kRowsMinPartition && pl.ps % kRowsTile == 0 && most_parts >= kRowsMinPartitions &&
      est_units >= kRowsWorkgroups && rows_head_group(d.num_kv_heads, G) >= 2 &&
      lgm::decode_rows_supported(act, cache, d.head_dim, d.num_kv_heads, G, d.block_size)) {
    // Whole-row kernel over equal runs of whole partitions, plain
    // ceil(L / ps) partitions (the ranges already balance the work).
    pl.rows = pl.rows_parts = true;
    pl.HG = rows_head_group(d.num_kv_heads, G);
    pl.parts = lgm::PartitionPlan{pl.ps, pl.ps};
    pl.P = pl.parts.max_count(max_ctx);
    const int64_t units = (int64_t)d.num_seqs * (d.num_kv_heads / pl.HG) * pl.P;
    if (units > (int64_t)INT32_MAX || (int64_t)d.num_seqs * d.num_q_heads > (int64_t)INT32_MAX - 1024)
      return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs * head groups * partitions = %lld: too many", (long long)units);
    pl.W = (int32_t)(units < 1 ? 1 : (units > kRowsWorkgroups ? kRowsWorkgroups : units));
    if (pl.P > 1) {
      pl.counters_bytes = kCounterSlot;
      pl.part_out_bytes = align256((size_t)d.num_seqs * d.num_q_heads * pl.P * d.head_dim * sizeof(float));
      pl.part_lse_bytes = align256((size_t)d.num_seqs * d.num_q_heads * pl.P * sizeof(float));
    }
    pl.total = pl.counters_bytes + pl.part_out_bytes + pl.part_lse_bytes;
    return LGM_OK;
  }
  // When contexts are split, the tokens past a context's last full partition
  // go to partitions of half the size, which the kernels take last: the work
  // drains on short items instead of ending on long ones.
  pl.parts = lgm::PartitionPlan{pl.ps, pl.ps};
  if (max_ctx > pl.ps) {
    const int32_t q = pl.ps / kTailDivisor / d.block_size * d.block_size;
    pl.parts.tps = q < d.block_size ? d.block_size : q;
  }
  pl.P = pl.parts.max_count(max_ctx);
  if (pl.P > 65535)  // the partition index is a grid dimension of the vector-ALU kernel
    return fail(LGM_ERR_UNSUPPORTED, fn, "max_context_len = %d / partition_size = %d gives %d partitions: at most 65535",
                max_ctx, pl.ps, pl.P);
  // Work item numbers of the persistent kernel are 32-bit, with room for one
  // overshooting fetch per workgroup.
  if (persistent && (int64_t)d.num_seqs * d.num_kv_heads * pl.P > (int64_t)INT32_MAX - (1 << 20))
    return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs * num_kv_heads * partitions = %lld work items: too many",
                (long long)d.num_seqs * d.num_kv_heads * pl.P);
  if (persistent || pl.P > 1) pl.counters_bytes = kCounterSlot;
  if (pl.P > 1) {
    pl.part_out_bytes = align256((size_t)d.num_seqs * d.num_q_heads * pl.P * d.head_dim * sizeof(float));
    pl.part_lse_bytes = align256((size_t)d.num_seqs * d.num_q_heads * pl.P * sizeof(float));
  }
  pl.total = pl.counters_bytes + pl.part_out_bytes + pl.part_lse_bytes;
  return LGM_OK;
}

lgm_status check_decode_common(const char* fn, const lgm_paged_dims& d, int32_t max_ctx, lgm_dtype cache) {
  lgm_status st = check_dims(fn, d);
  if (st != LGM_OK) return st;
  if (!dtype_valid(cache)) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "cache_dtype = %d is not an lgm_dtype", (int)cache);
  const int64_t cap = (int64_t)d.max_blocks_per_seq * d.block_size;
  if (max_ctx < 0 || max_ctx > cap)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn,
                "max_context_len = %d must be in [0, max_blocks_per_seq * block_size = %lld]", max_ctx, (long long)cap);
  return LGM_OK;
}

// ---- paged MLA ------------------------------------------------------------------
// Auto partition of the MLA kernel: about one workgroup (a partition of one
// sequence, its four waves taking turns over the 32-token tiles) per compute
// unit of MI355X at max_context_len, and at least one tile per wave.
constexpr int64_t kMlaTargetWorkgroups = 256;
constexpr int32_t kMlaTile = 32;
constexpr int32_t kMlaAutoStep = 64;  // the kernel's tile: a partition's last tile costs a whole tile
constexpr int32_t kMlaMinAutoPartition = 128;

lgm_status check_mla_dims(const char* fn, const lgm_mla_dims& d, int32_t max_ctx) {
  if (d.num_seqs < 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_seqs = %d must be >= 0", d.num_seqs);
  if (d.num_heads < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_heads = %d must be >= 1", d.num_heads);
  if (d.latent_dim < 1 || d.rope_dim < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.latent_dim = %d and dims.rope_dim = %d must be >= 1",
                d.latent_dim, d.rope_dim);
  if (d.block_size < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.block_size = %d must be >= 1", d.block_size);
  if (d.num_blocks < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.num_blocks = %d must be >= 1", d.num_blocks);
  if (d.max_blocks_per_seq < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.max_blocks_per_seq = %d must be >= 1", d.max_blocks_per_seq);
  const int64_t cap = (int64_t)d.max_blocks_per_seq * d.block_size;
  if (cap > INT32_MAX)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "dims.max_blocks_per_seq * dims.block_size = %lld exceeds INT32_MAX",
                (long long)cap);
  if (max_ctx < 0 || max_ctx > cap)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn,
                "max_context_len = %d must be in [0, max_blocks_per_seq * block_size = %lld]", max_ctx, (long long)cap);
  if (!lgm::mla_supported(LGM_FP8_E4M3, d.latent_dim, d.rope_dim, d.num_heads, d.block_size))
    return fail(LGM_ERR_UNSUPPORTED, fn,
                "(latent_dim %d, rope_dim %d, num_heads %d, block_size %d) unsupported: supported are latent_dim "
                "512, rope_dim 64, num_heads 1..16, block_size a power of two",
                d.latent_dim, d.rope_dim, d.num_heads, d.block_size);
  if (d.num_seqs > 65535) return fail(LGM_ERR_UNSUPPORTED, fn, "dims.num_seqs = %d: at most 65535", d.num_seqs);
  if ((int64_t)d.num_seqs * d.num_heads > (int64_t)INT32_MAX - 1024)  // merge rows are int-indexed
    return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs * num_heads = %lld: too many",
                (long long)d.num_seqs * d.num_heads);
  return LGM_OK;
}

struct MlaPlan {
  int32_t ps, P;
  size_t part_out_bytes, part_lse_bytes, total;
};

lgm_status plan_mla(const char* fn, const lgm_mla_dims& d, int32_t max_ctx, int32_t ps, MlaPlan& pl) {
  pl = MlaPlan{};
  if (ps < 0 || ps % kMlaTile != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "partition_size = %d must be 0 (library chooses) or a positive "
                "multiple of %d", ps, kMlaTile);
  const int64_t cap = ((int64_t)(max_ctx > 0 ? max_ctx : 1) + kMlaTile - 1) / kMlaTile * kMlaTile;
  int64_t p = ps;
  if (p == 0) {
    const int64_t tokens = (int64_t)(d.num_seqs > 0 ? d.num_seqs : 1) * max_ctx;
    p = (tokens + kMlaTargetWorkgroups - 1) / kMlaTargetWorkgroups;
    p = (p + kMlaAutoStep - 1) / kMlaAutoStep * kMlaAutoStep;
    p = p < kMlaMinAutoPartition ? kMlaMinAutoPartition : p;
  }
  pl.ps = (int32_t)(p < cap ? p : cap);
  pl.P = (int32_t)(((int64_t)max_ctx + pl.ps - 1) / pl.ps);
  pl.P = pl.P < 1 ? 1 : pl.P;
  if (pl.P > 1) {
    pl.part_out_bytes = align256((size_t)d.num_seqs * d.num_heads * pl.P * d.latent_dim * sizeof(float));
    pl.part_lse_bytes = align256((size_t)d.num_seqs * d.num_heads * pl.P * sizeof(float));
  }
  pl.total = pl.part_out_bytes + pl.part_lse_bytes;
  return LGM_OK;
}

}  // namespace

extern "C" {

const char* lgm_last_error(void) { return g_err.c_str(); }

int32_t lgm_abi_version(void) { return LGM_ABI_VERSION; }

lgm_status lgm_rope_kv_append(const void* qkv, int64_t qkv_row_stride, void* q_out, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                              const float* v_scale, float rope_theta, lgm_paged_dims dims, lgm_dtype act_dtype,
                              lgm_dtype cache_dtype, uint32_t flags, void* stream) {
  const char* fn = "lgm_rope_kv_append";
  g_err.clear();
  lgm_status st = check_dims(fn, dims);
  if (st != LGM_OK) return st;
  if (dims.head_dim > 256)
    return fail(LGM_ERR_UNSUPPORTED, fn, "dims.head_dim = %d: supported head_dim is even, 2..256", dims.head_dim);
  if (!dtype_valid(act_dtype)) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "act_dtype = %d is not an lgm_dtype", (int)act_dtype);
  if (!dtype_valid(cache_dtype))
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "cache_dtype = %d is not an lgm_dtype", (int)cache_dtype);
  const bool types_ok = (act_dtype == LGM_F32 && cache_dtype == LGM_F32) ||
                        (act_dtype == LGM_BF16 && cache_dtype == LGM_BF16) ||
                        (act_dtype == LGM_BF16 && cache_dtype == LGM_FP8_E4M3) ||
                        (act_dtype == LGM_BF16 && cache_dtype == LGM_FP4_E2M1);
  if (!types_ok)
    return fail(LGM_ERR_UNSUPPORTED, fn, "(act_dtype, cache_dtype) = (%s, %s): supported are (F32, F32), "
                "(BF16, BF16), (BF16, FP8_E4M3), (BF16, FP4_E2M1)", dtype_name(act_dtype), dtype_name(cache_dtype));
  if (cache_dtype == LGM_FP4_E2M1 && dims.head_dim % 32 != 0)
    return fail(LGM_ERR_UNSUPPORTED, fn, "dims.head_dim = %d: FP4 caches need a multiple of 32 (one scale per 32)",
                dims.head_dim);
  if (!(std::isfinite(rope_theta) && rope_theta > 0.f))
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "rope_theta = %g must be finite and > 0", (double)rope_theta);
  const int64_t row = (int64_t)(dims.num_q_heads + 2 * dims.num_kv_heads) * dims.head_dim;
  if (qkv_row_stride < row)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "qkv_row_stride = %lld must be >= (Hq + 2*Hkv) * D = %lld",
                (long long)qkv_row_stride, (long long)row);
  if ((st = check_scales(fn, cache_dtype, k_scale, v_scale)) != LGM_OK) return st;
  if ((st = check_flags(fn, flags, LGM_ROPE_INTERLEAVED | LGM_CACHE_HND | LGM_SCALE_PER_TENSOR, cache_dtype)) !=
      LGM_OK)
    return st;
  if (dims.num_seqs == 0) return LGM_OK;
  if (!qkv) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "qkv is NULL");
  if (!q_out) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "q_out is NULL");
  if (!k_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "k_cache is NULL");
  if (!v_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "v_cache is NULL");
  if (!block_tables) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "block_tables is NULL");
  if (!context_lens) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "context_lens is NULL");

  const int64_t ea = elem_bytes(act_dtype);
  const int64_t B = dims.num_seqs;
  const Span outs[] = {{"q_out", (uintptr_t)q_out, B * dims.num_q_heads * dims.head_dim * ea},
                       {"k_cache", (uintptr_t)k_cache, cache_bytes(dims, cache_dtype)},
                       {"v_cache", (uintptr_t)v_cache, cache_bytes(dims, cache_dtype)}};
  const Span ins[] = {{"qkv", (uintptr_t)qkv, ((B - 1) * qkv_row_stride + row) * ea},
                      {"block_tables", (uintptr_t)block_tables, B * dims.max_blocks_per_seq * 4},
                      {"context_lens", (uintptr_t)context_lens, B * 4},
                      {"k_scale", (uintptr_t)k_scale, scale_bytes(k_scale, dims, flags)},
                      {"v_scale", (uintptr_t)v_scale, scale_bytes(v_scale, dims, flags)}};
  if ((st = check_no_alias(fn, outs, 3, ins, 5)) != LGM_OK) return st;

  lgm::AppendArgs a{qkv, qkv_row_stride, q_out, k_cache, v_cache, block_tables, context_lens,
                    k_scale, v_scale, rope_theta, dims, flags};
  const hipError_t e = lgm::launch_rope_kv_append(a, act_dtype, cache_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
  return LGM_OK;
}

int32_t lgm_paged_decode_partition_size(lgm_paged_dims dims, int32_t max_context_len, int32_t partition_size,
                                        lgm_dtype cache_dtype) {
  const char* fn = "lgm_paged_decode_partition_size";
  g_err.clear();
  if (check_decode_common(fn, dims, max_context_len, cache_dtype) != LGM_OK) return -1;
  Plan pl;
  if (plan_decode(fn, dims, max_context_len, partition_size, cache_dtype, pl) != LGM_OK) return -1;
  return pl.rows && !pl.rows_parts ? 0 : pl.ps;
}

size_t lgm_paged_decode_workspace_size(lgm_paged_dims dims, int32_t max_context_len, int32_t partition_size,
                                       lgm_dtype cache_dtype) {
  const char* fn = "lgm_paged_decode_workspace_size";
  g_err.clear();
  if (check_decode_common(fn, dims, max_context_len, cache_dtype) != LGM_OK) return 0;
  Plan pl;
  if (plan_decode(fn, dims, max_context_len, partition_size, cache_dtype, pl) != LGM_OK) return 0;
  return pl.total;
}

}  // extern "C"

namespace {

// Where lgm_paged_decode_attn_static finds its workspace.
struct StaticWorkspace {
  void* ptr;
  size_t bytes;
};
constexpr size_t kStaticScratchBytes = LGM_STATIC_SCRATCH_BYTES;
using ScratchResolver = lgm_status (*)(const char* fn, hipStream_t stream, StaticWorkspace& sw);

// The attention call of both entry points.  resolve_static is NULL for
// lgm_paged_decode_attn (the caller's workspace is checked and used);
// lgm_paged_decode_attn_static passes the resolver of the device-resident
// scratch array, called only after every other argument has been validated.
lgm_status decode_attn_impl(const char* fn, void* out, float* out_lse, const void* q, int64_t q_seq_stride,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const float* k_scale, const float* v_scale,
                            float softmax_scale, int32_t partition_size, int32_t max_context_len, void* workspace,
                            size_t workspace_bytes, lgm_paged_dims dims, lgm_dtype act_dtype, lgm_dtype cache_dtype,
                            uint32_t flags, void* stream, ScratchResolver resolve_static) {
  lgm_status st = check_decode_common(fn, dims, max_context_len, cache_dtype);
  if (st != LGM_OK) return st;
  if (!dtype_valid(act_dtype)) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "act_dtype = %d is not an lgm_dtype", (int)act_dtype);
  const int G = dims.num_q_heads / dims.num_kv_heads;
  if (!lgm::decode_supported(act_dtype, cache_dtype, dims.head_dim, G, dims.block_size))
    return fail(LGM_ERR_UNSUPPORTED, fn,
                "(act %s, cache %s, head_dim %d, group %d, block_size %d) unsupported: supported are (F32, F32), "
                "(BF16, BF16), (BF16, FP8_E4M3) with head_dim 64 or 128, block_size 16, group 1..8 "
                "(1..16 for bf16 activations at head_dim 128), and (BF16, FP4_E2M1) with head_dim 128, "
                "block_size 16, group 1..16",
                dtype_name(act_dtype), dtype_name(cache_dtype), dims.head_dim, G, dims.block_size);
  if (dims.num_seqs > 65535 || dims.num_kv_heads > 65535)
    return fail(LGM_ERR_UNSUPPORTED, fn, "dims.num_seqs = %d / dims.num_kv_heads = %d: at most 65535 each",
                dims.num_seqs, dims.num_kv_heads);
  if (!std::isfinite(softmax_scale))
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "softmax_scale = %g must be finite", (double)softmax_scale);
  const int64_t qrow = (int64_t)dims.num_q_heads * dims.head_dim;
  if (q_seq_stride < qrow)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "q_seq_stride = %lld must be >= num_q_heads * head_dim = %lld",
                (long long)q_seq_stride, (long long)qrow);
  if ((st = check_scales(fn, cache_dtype, k_scale, v_scale)) != LGM_OK) return st;
  if ((st = check_flags(fn, flags, LGM_CACHE_HND | LGM_SCALE_PER_TENSOR, cache_dtype)) != LGM_OK) return st;
  Plan pl;
  if ((st = plan_decode(fn, dims, max_context_len, partition_size, cache_dtype, pl)) != LGM_OK) return st;
  struct {
    size_t total;
  } ws{pl.total};
  if (resolve_static && ws.total > kStaticScratchBytes)
    return fail(LGM_ERR_WORKSPACE_TOO_SMALL, fn,
                "these arguments need %zu bytes of workspace, more than the %zu bytes of the device-resident scratch "
                "array (LGM_STATIC_SCRATCH_BYTES); call lgm_paged_decode_attn with a workspace instead",
                ws.total, (size_t)kStaticScratchBytes);
  if (ws.total > 0 && !resolve_static) {
    if (!workspace)
      return fail(LGM_ERR_WORKSPACE_TOO_SMALL, fn, "workspace is NULL but %zu bytes are needed", ws.total);
    if (workspace_bytes < ws.total)
      return fail(LGM_ERR_WORKSPACE_TOO_SMALL, fn, "workspace_bytes = %zu < %zu needed", workspace_bytes, ws.total);
    if ((uintptr_t)workspace % 256 != 0)
      return fail(LGM_ERR_INVALID_ARGUMENT, fn, "workspace %p must be 256-byte aligned", workspace);
  }
  if (dims.num_seqs == 0) return LGM_OK;
  if (!out) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "out is NULL");
  if (!q) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "q is NULL");
  if (!k_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "k_cache is NULL");
  if (!v_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "v_cache is NULL");
  if (!block_tables) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "block_tables is NULL");
  if (!context_lens) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "context_lens is NULL");
  if ((uintptr_t)k_cache % 16 != 0 || (uintptr_t)v_cache % 16 != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "k_cache (%p) and v_cache (%p) must be 16-byte aligned", k_cache, v_cache);
  if ((uintptr_t)out % 16 != 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "out (%p) must be 16-byte aligned", out);

  const int64_t ea = elem_bytes(act_dtype);
  const int64_t B = dims.num_seqs;
  const Span outs[] = {{"out", (uintptr_t)out, B * qrow * ea},
                       {"out_lse", (uintptr_t)out_lse, out_lse ? B * dims.num_q_heads * 4 : 0},
                       {"workspace", (uintptr_t)workspace, (int64_t)ws.total}};
  const Span ins[] = {{"q", (uintptr_t)q, ((B - 1) * q_seq_stride + qrow) * ea},
                      {"k_cache", (uintptr_t)k_cache, cache_bytes(dims, cache_dtype)},
                      {"v_cache", (uintptr_t)v_cache, cache_bytes(dims, cache_dtype)},
                      {"block_tables", (uintptr_t)block_tables, B * dims.max_blocks_per_seq * 4},
                      {"context_lens", (uintptr_t)context_lens, B * 4},
                      {"k_scale", (uintptr_t)k_scale, scale_bytes(k_scale, dims, flags)},
                      {"v_scale", (uintptr_t)v_scale, scale_bytes(v_scale, dims, flags)}};
  if ((st = check_no_alias(fn, outs, 3, ins, 7)) != LGM_OK) return st;

  if (resolve_static) {
    StaticWorkspace sw{};
    if ((st = resolve_static(fn, (hipStream_t)stream, sw)) != LGM_OK) return st;
    workspace = sw.ptr;
    workspace_bytes = sw.bytes;
  }
  char* wsb = static_cast<char*>(workspace);
  if (pl.fused) {
    lgm::DecodeArgs a{out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                      nullptr, nullptr, nullptr, softmax_scale, lgm::PartitionPlan{pl.ps, pl.ps}, max_context_len,
                      pl.P, dims, flags};
    lgm::FusedArgs f{};
    f.chunk_steps = pl.chunk_steps;
    f.nchunks = pl.nchunks;
    f.rec_out = pl.rec_out_bytes ? reinterpret_cast<float*>(wsb + pl.counters_bytes) : nullptr;
    f.rec_lse = pl.rec_lse_bytes ? reinterpret_cast<float*>(wsb + pl.counters_bytes + pl.rec_out_bytes) : nullptr;
    f.rec_out_bytes = (int32_t)pl.rec_out_bytes;
    f.rec_lse_bytes = (int32_t)pl.rec_lse_bytes;
    f.arrivals = reinterpret_cast<int32_t*>(wsb) + 2;
    const hipError_t e = lgm::launch_paged_decode_fused(a, f, cache_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "single-launch kernel launch failed: %s", hipGetErrorString(e));
    return LGM_OK;
  }
  if (pl.rows_parts) {
    float* part_out = pl.P > 1 ? reinterpret_cast<float*>(wsb + pl.counters_bytes) : nullptr;
    float* part_lse = pl.P > 1 ? reinterpret_cast<float*>(wsb + pl.counters_bytes + pl.part_out_bytes) : nullptr;
    lgm::DecodeArgs a{out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                      part_out, part_lse, nullptr, softmax_scale, pl.parts, max_context_len, pl.P, dims, flags};
    lgm::RowsArgs r{};
    r.num_wg = pl.W;
    r.head_group = pl.HG;
    r.part_tiles = pl.ps / (int32_t)kRowsTile;
    hipError_t e = lgm::launch_paged_decode_rows(a, r, cache_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "row kernel launch failed: %s", hipGetErrorString(e));
    if (pl.P > 1) {
      lgm::MergeArgs m{out, out_lse, part_out, part_lse, nullptr, context_lens, pl.parts, max_context_len,
                       dims.num_seqs, dims.num_q_heads, dims.head_dim, pl.P, 1};
      e = lgm::launch_lse_merge(m, act_dtype, (hipStream_t)stream);
      if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "merge kernel launch failed: %s", hipGetErrorString(e));
    }
    return LGM_OK;
  }
  if (pl.rows) {
    lgm::DecodeArgs a{out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                      nullptr, nullptr, nullptr, softmax_scale, lgm::PartitionPlan{1, 1}, max_context_len, 0, dims,
                      flags};
    char* w = wsb + pl.counters_bytes;
    lgm::RowsArgs r{};
    r.num_wg = pl.W;
    r.head_group = pl.HG;
    r.rec_out = reinterpret_cast<float*>(w);
    w += pl.rec_out_bytes;
    r.rec_lse = reinterpret_cast<float*>(w);
    w += pl.rec_lse_bytes;
    r.wg_first = reinterpret_cast<int32_t*>(w);
    w += pl.stream_bytes;
    r.wg_last = reinterpret_cast<int32_t*>(w);
    const hipError_t e = lgm::launch_paged_decode_rows(a, r, cache_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "row kernel launch failed: %s", hipGetErrorString(e));
    return LGM_OK;
  }
  int32_t* counters = pl.counters_bytes && lgm::decode_mfma_supported(act_dtype, cache_dtype, dims.head_dim, G,
                                                                     dims.block_size)
                          ? reinterpret_cast<int32_t*>(wsb)
                          : nullptr;
  float* part_out = pl.P > 1 ? reinterpret_cast<float*>(wsb + pl.counters_bytes) : nullptr;
  float* part_lse = pl.P > 1 ? reinterpret_cast<float*>(wsb + pl.counters_bytes + pl.part_out_bytes) : nullptr;
  lgm::DecodeArgs a{out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                    part_out, part_lse, counters, softmax_scale, pl.parts, max_context_len, pl.P, dims, flags};
  hipError_t e = lgm::launch_paged_decode(a, act_dtype, cache_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "split kernel launch failed: %s", hipGetErrorString(e));
  if (pl.P > 1) {
    lgm::MergeArgs m{out, out_lse, part_out, part_lse, nullptr, context_lens, pl.parts, max_context_len,
                     dims.num_seqs, dims.num_q_heads, dims.head_dim, pl.P, 1};
    e = lgm::launch_lse_merge(m, act_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "merge kernel launch failed: %s", hipGetErrorString(e));
  }
  return LGM_OK;
}

// ---- the device-resident scratch array of lgm_paged_decode_attn_static -----------
// One copy per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address: each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchWords = kStaticScratchBytes / 4;
static __device__ __align__(256) uint32_t scratch[kStaticScratchWords];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  hipError_t err;
  void* ptr;
};
ScratchSlot g_scratch[kMaxDevices];

// The scratch array of the device `stream` runs on.  The first call on a
// device looks its address up (with that device current) and clears the
// work-counter slot at its start with a small kernel on `stream` (a kernel,
// not a memset, so that a caller capturing a graph records an ordinary
// node); every completed call leaves that slot zero again.
lgm_status resolve_scratch(const char* fn, hipStream_t stream, StaticWorkspace& sw) {
  int dev = 0;
  if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
    if (hipGetDevice(&dev) != hipSuccess) return fail(LGM_ERR_HIP, fn, "hipGetDevice failed");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LGM_ERR_UNSUPPORTED, fn, "device %d: the scratch array is kept for devices 0..%d", dev,
                kMaxDevices - 1);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    int cur = -1;
    slot.err = hipGetDevice(&cur);
    if (slot.err != hipSuccess) return;
    if (cur != dev && (slot.err = hipSetDevice(dev)) != hipSuccess) return;
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (slot.err == hipSuccess) {
      slot.ptr = p;
      constexpr int kWords = (int)(kCounterSlot / 4);
      hipLaunchKernelGGL(zero_words_kernel, dim3((kWords + 255) / 256), dim3(256), 0, stream,
                         static_cast<uint32_t*>(p), kWords);
      slot.err = hipGetLastError();
    }
    if (cur != dev) {
      const hipError_t e = hipSetDevice(cur);
      if (slot.err == hipSuccess) slot.err = e;
    }
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr)
    return fail(LGM_ERR_HIP, fn, "device %d: the scratch array's address could not be taken: %s", dev,
                hipGetErrorString(slot.err));
  sw.ptr = slot.ptr;
  sw.bytes = kStaticScratchBytes;
  return LGM_OK;
}

}  // namespace

extern "C" {

lgm_status lgm_paged_decode_attn(void* out, float* out_lse, const void* q, int64_t q_seq_stride, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                 const float* k_scale, const float* v_scale, float softmax_scale,
                                 int32_t partition_size, int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, lgm_paged_dims dims, lgm_dtype act_dtype,
                                 lgm_dtype cache_dtype, uint32_t flags, void* stream) {
  g_err.clear();
  return decode_attn_impl("lgm_paged_decode_attn", out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables,
                          context_lens, k_scale, v_scale, softmax_scale, partition_size, max_context_len, workspace,
                          workspace_bytes, dims, act_dtype, cache_dtype, flags, stream, nullptr);
}

lgm_status lgm_paged_decode_attn_static(void* out, float* out_lse, const void* q, int64_t q_seq_stride,
                                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, const float* k_scale, const float* v_scale,
                                        float softmax_scale, int32_t partition_size, int32_t max_context_len,
                                        lgm_paged_dims dims, lgm_dtype act_dtype, lgm_dtype cache_dtype,
                                        uint32_t flags, void* stream) {
  g_err.clear();
  return decode_attn_impl("lgm_paged_decode_attn_static", out, out_lse, q, q_seq_stride, k_cache, v_cache,
                          block_tables, context_lens, k_scale, v_scale, softmax_scale, partition_size,
                          max_context_len, nullptr, 0, dims, act_dtype, cache_dtype, flags, stream, resolve_scratch);
}

lgm_status lgm_check_block_tables(const int32_t* block_tables, const int32_t* context_lens, lgm_paged_dims dims,
                                  int32_t max_context_len, int32_t* status, void* stream) {
  const char* fn = "lgm_check_block_tables";
  g_err.clear();
  lgm_status st = check_dims(fn, dims);
  if (st != LGM_OK) return st;
  const int64_t cap = (int64_t)dims.max_blocks_per_seq * dims.block_size;
  if (max_context_len < 0 || max_context_len > cap)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn,
                "max_context_len = %d must be in [0, max_blocks_per_seq * block_size = %lld]", max_context_len,
                (long long)cap);
  if (dims.num_seqs > 65535) return fail(LGM_ERR_UNSUPPORTED, fn, "dims.num_seqs = %d: at most 65535", dims.num_seqs);
  if (dims.num_seqs == 0) return LGM_OK;
  if (!block_tables) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "block_tables is NULL");
  if (!context_lens) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "context_lens is NULL");
  if (!status) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "status is NULL");
  if ((uintptr_t)status % 4 != 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "status %p must be 4-byte aligned", (void*)status);
  const int64_t B = dims.num_seqs;
  const Span outs[] = {{"status", (uintptr_t)status, 16}};
  const Span ins[] = {{"block_tables", (uintptr_t)block_tables, B * dims.max_blocks_per_seq * 4},
                      {"context_lens", (uintptr_t)context_lens, B * 4}};
  if ((st = check_no_alias(fn, outs, 1, ins, 2)) != LGM_OK) return st;
  const hipError_t e =
      lgm::launch_table_check(block_tables, context_lens, dims, max_context_len, status, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
  return LGM_OK;
}

lgm_status lgm_lse_merge(void* out, float* out_lse, const float* partial_out, const float* partial_lse,
                         const int32_t* num_partitions, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                         int32_t max_partitions, lgm_dtype out_dtype, void* stream) {
  const char* fn = "lgm_lse_merge";
  g_err.clear();
  if (num_seqs < 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "num_seqs = %d must be >= 0", num_seqs);
  if (num_q_heads < 1) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "num_q_heads = %d must be >= 1", num_q_heads);
  if (max_partitions < 1)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "max_partitions = %d must be >= 1", max_partitions);
  if (!(out_dtype == LGM_F32 || out_dtype == LGM_BF16))
    return fail(LGM_ERR_UNSUPPORTED, fn, "out_dtype = %d: supported are LGM_F32 and LGM_BF16", (int)out_dtype);
  if (!lgm::merge_supported(head_dim))
    return fail(LGM_ERR_UNSUPPORTED, fn, "head_dim = %d: supported are 64, 128 and 512", head_dim);
  if (num_seqs > 65535)
    return fail(LGM_ERR_UNSUPPORTED, fn, "num_seqs = %d: at most 65535", num_seqs);
  if (num_seqs == 0) return LGM_OK;
  if (!out) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "out is NULL");
  if (!partial_out) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "partial_out is NULL");
  if (!partial_lse) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "partial_lse is NULL");
  if ((uintptr_t)partial_out % 16 != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "partial_out %p must be 16-byte aligned", (const void*)partial_out);
  const int64_t rows = (int64_t)num_seqs * num_q_heads;
  const Span outs[] = {{"out", (uintptr_t)out, rows * head_dim * elem_bytes(out_dtype)},
                       {"out_lse", (uintptr_t)out_lse, out_lse ? rows * 4 : 0}};
  const Span ins[] = {{"partial_out", (uintptr_t)partial_out, rows * max_partitions * head_dim * 4},
                      {"partial_lse", (uintptr_t)partial_lse, rows * max_partitions * 4},
                      {"num_partitions", (uintptr_t)num_partitions, num_partitions ? (int64_t)num_seqs * 4 : 0}};
  lgm_status st = check_no_alias(fn, outs, 2, ins, 3);
  if (st != LGM_OK) return st;
  lgm::MergeArgs m{out, out_lse, partial_out, partial_lse, num_partitions, nullptr, lgm::PartitionPlan{1, 1}, 0,
                   num_seqs, num_q_heads, head_dim, max_partitions, 0};
  const hipError_t e = lgm::launch_lse_merge(m, out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
  return LGM_OK;
}

int32_t lgm_paged_mla_partition_size(lgm_mla_dims dims, int32_t max_context_len, int32_t partition_size) {
  const char* fn = "lgm_paged_mla_partition_size";
  g_err.clear();
  if (check_mla_dims(fn, dims, max_context_len) != LGM_OK) return -1;
  MlaPlan pl;
  if (plan_mla(fn, dims, max_context_len, partition_size, pl) != LGM_OK) return -1;
  return pl.ps;
}

size_t lgm_paged_mla_workspace_size(lgm_mla_dims dims, int32_t max_context_len, int32_t partition_size) {
  const char* fn = "lgm_paged_mla_workspace_size";
  g_err.clear();
  if (check_mla_dims(fn, dims, max_context_len) != LGM_OK) return 0;
  MlaPlan pl;
  if (plan_mla(fn, dims, max_context_len, partition_size, pl) != LGM_OK) return 0;
  return pl.total;
}

lgm_status lgm_paged_mla_decode(void* out, float* out_lse, const void* q_latent, const void* q_pe,
                                const void* ckv_cache, const void* kpe_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const float* ckv_scale, float softmax_scale,
                                int32_t partition_size, int32_t max_context_len, void* workspace,
                                size_t workspace_bytes, lgm_mla_dims dims, lgm_dtype ckv_dtype, void* stream) {
  const char* fn = "lgm_paged_mla_decode";
  g_err.clear();
  lgm_status st = check_mla_dims(fn, dims, max_context_len);
  if (st != LGM_OK) return st;
  if (!dtype_valid(ckv_dtype)) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "ckv_dtype = %d is not an lgm_dtype", (int)ckv_dtype);
  if (ckv_dtype != LGM_FP8_E4M3)
    return fail(LGM_ERR_UNSUPPORTED, fn, "ckv_dtype = %s: supported is LGM_FP8_E4M3", dtype_name(ckv_dtype));
  if (!std::isfinite(softmax_scale))
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "softmax_scale = %g must be finite", (double)softmax_scale);
  MlaPlan pl;
  if ((st = plan_mla(fn, dims, max_context_len, partition_size, pl)) != LGM_OK) return st;
  if (pl.total > 0) {
    if (!workspace)
      return fail(LGM_ERR_WORKSPACE_TOO_SMALL, fn, "workspace is NULL but %zu bytes are needed", pl.total);
    if (workspace_bytes < pl.total)
      return fail(LGM_ERR_WORKSPACE_TOO_SMALL, fn, "workspace_bytes = %zu < %zu needed", workspace_bytes, pl.total);
    if ((uintptr_t)workspace % 256 != 0)
      return fail(LGM_ERR_INVALID_ARGUMENT, fn, "workspace %p must be 256-byte aligned", workspace);
  }
  if (!ckv_scale) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "ckv_scale is NULL; an FP8 ckv cache needs its fp32 [1] scale");
  if (dims.num_seqs == 0) return LGM_OK;
  if (!out) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "out is NULL");
  if (!q_latent) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "q_latent is NULL");
  if (!q_pe) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "q_pe is NULL");
  if (!ckv_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "ckv_cache is NULL");
  if (!kpe_cache) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "kpe_cache is NULL");
  if (!block_tables) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "block_tables is NULL");
  if (!context_lens) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "context_lens is NULL");
  const void* aligned[] = {out, q_latent, q_pe, ckv_cache, kpe_cache};
  const char* aligned_names[] = {"out", "q_latent", "q_pe", "ckv_cache", "kpe_cache"};
  for (int i = 0; i < 5; ++i)
    if ((uintptr_t)aligned[i] % 16 != 0)
      return fail(LGM_ERR_INVALID_ARGUMENT, fn, "%s (%p) must be 16-byte aligned", aligned_names[i], aligned[i]);

  const int64_t B = dims.num_seqs, H = dims.num_heads;
  const int64_t pool_rows = (int64_t)dims.num_blocks * dims.block_size;
  const Span outs[] = {{"out", (uintptr_t)out, B * H * dims.latent_dim * 2},
                       {"out_lse", (uintptr_t)out_lse, out_lse ? B * H * 4 : 0},
                       {"workspace", (uintptr_t)workspace, (int64_t)pl.total}};
  const Span ins[] = {{"q_latent", (uintptr_t)q_latent, B * H * dims.latent_dim * 2},
                      {"q_pe", (uintptr_t)q_pe, B * H * dims.rope_dim * 2},
                      {"ckv_cache", (uintptr_t)ckv_cache, pool_rows * dims.latent_dim},
                      {"kpe_cache", (uintptr_t)kpe_cache, pool_rows * dims.rope_dim * 2},
                      {"block_tables", (uintptr_t)block_tables, B * dims.max_blocks_per_seq * 4},
                      {"context_lens", (uintptr_t)context_lens, B * 4},
                      {"ckv_scale", (uintptr_t)ckv_scale, 4}};
  if ((st = check_no_alias(fn, outs, 3, ins, 7)) != LGM_OK) return st;

  char* wsb = static_cast<char*>(workspace);
  float* part_out = pl.P > 1 ? reinterpret_cast<float*>(wsb) : nullptr;
  float* part_lse = pl.P > 1 ? reinterpret_cast<float*>(wsb + pl.part_out_bytes) : nullptr;
  lgm::MlaArgs a{out, out_lse, q_latent, q_pe, ckv_cache, kpe_cache, block_tables, context_lens, ckv_scale,
                 part_out, part_lse, softmax_scale, pl.ps, max_context_len, pl.P, dims};
  hipError_t e = lgm::launch_paged_mla(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "MLA kernel launch failed: %s", hipGetErrorString(e));
  if (pl.P > 1) {
    lgm::MergeArgs m{out, out_lse, part_out, part_lse, nullptr, context_lens, lgm::PartitionPlan{pl.ps, pl.ps},
                     max_context_len, dims.num_seqs, dims.num_heads, dims.latent_dim, pl.P, 1};
    e = lgm::launch_lse_merge(m, LGM_BF16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "merge kernel launch failed: %s", hipGetErrorString(e));
  }
  return LGM_OK;
}

lgm_status lgm_stream_read_probe(const void* src, size_t bytes, int32_t num_workgroups, int32_t nontemporal,
                                 uint32_t* sink, void* stream) {
  const char* fn = "lgm_stream_read_probe";
  g_err.clear();
  if (!src) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "src is NULL");
  if (!sink) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "sink is NULL");
  if ((uintptr_t)src % 16 != 0) return fail(LGM_ERR_INVALID_ARGUMENT, fn, "src %p must be 16-byte aligned", src);
  if (num_workgroups < 1 || num_workgroups > 65536)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "num_workgroups = %d must be in [1, 65536]", num_workgroups);
  const uint64_t unit = (uint64_t)num_workgroups * lgm::stream_probe_granule();
  if (bytes == 0 || bytes % unit != 0)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "bytes = %zu must be a positive multiple of num_workgroups * %d = %llu",
                bytes, lgm::stream_probe_granule(), (unsigned long long)unit);
  if (bytes / num_workgroups > (uint64_t)INT32_MAX)
    return fail(LGM_ERR_INVALID_ARGUMENT, fn, "bytes / num_workgroups = %llu exceeds INT32_MAX",
                (unsigned long long)(bytes / num_workgroups));
  const Span outs[] = {{"sink", (uintptr_t)sink, 4}};
  const Span ins[] = {{"src", (uintptr_t)src, (int64_t)bytes}};
  lgm_status st = check_no_alias(fn, outs, 1, ins, 1);
  if (st != LGM_OK) return st;
  const hipError_t e =
      lgm::launch_stream_read_probe(src, (int64_t)bytes, num_workgroups, nontemporal != 0, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LGM_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
  return LGM_OK;
}

}  // extern "C"
