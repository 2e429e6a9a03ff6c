// Internal interface between the C-ABI host layer (lgm_api.cpp) and the
// kernel translation units.  Arguments reaching a launcher have already been
// validated by the host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lgm.h"
#include "lgm_mla.h"

namespace lgm {

constexpr int kWaveSize = 64;
constexpr int kDecodeThreads = 256;  // 4 waves per workgroup

struct AppendArgs {
  const void* qkv;
  int64_t qkv_row_stride;
  void* q_out;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  float rope_theta;
  lgm_paged_dims dims;
  uint32_t flags;  // LGM_ROPE_INTERLEAVED | LGM_CACHE_HND | LGM_SCALE_PER_TENSOR
};

// How one context of ctx tokens is cut into split-K partitions: the first
// nfull(ctx) = floor(ctx / ps) partitions hold ps tokens each, the rest of
// the context follows in partitions of tps <= ps tokens; an empty context has
// one (empty) partition.  {ps, ps} gives the plain ceil(ctx / ps) partitions.
struct PartitionPlan {
  int32_t ps, tps;
  __host__ __device__ int nfull(int ctx) const { return ctx / ps; }
  __host__ __device__ int count(int ctx) const {
    if (ctx <= 0) return 1;
    const int nf = nfull(ctx);
    return nf + (ctx - nf * ps + tps - 1) / tps;
  }
  __host__ __device__ void range(int ctx, int part, int& start, int& end) const {
    const int nf = nfull(ctx);
    if (part < nf) {
      start = part * ps;
      end = start + ps;
    } else {
      start = nf * ps + (part - nf) * tps;
      end = start + tps < ctx ? start + tps : ctx;
    }
  }
  // Largest count over contexts 0..max_ctx: count grows with ctx between
  // multiples of ps and drops at each multiple, so it peaks at max_ctx or
  // just below the largest multiple of ps not above it.
  __host__ __device__ int max_count(int max_ctx) const {
    int m = count(max_ctx);
    if (max_ctx >= ps) {
      const int below = count(max_ctx / ps * ps - 1);
      m = below > m ? below : m;
    }
    return m;
  }
};

struct DecodeArgs {
  void* out;
  float* out_lse;
  const void* q;
  int64_t q_seq_stride;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  float* part_out;   // [B][Hq][P][D] fp32, NULL when P == 1
  float* part_lse;   // [B][Hq][P] fp32
  int32_t* work_counters;  // matrix-core kernel: 2 ints, zero on entry, left zero on completion
  float softmax_scale;
  PartitionPlan parts;
  int32_t max_context_len;
  int32_t max_partitions;
  lgm_paged_dims dims;
  uint32_t flags;  // LGM_CACHE_HND | LGM_SCALE_PER_TENSOR
};

// Strides, in storage units, of a cache pool whose (token, kv head) rows are
// `row` units long: NHD blocks are [block_size][Hkv][row], HND blocks
// [Hkv][block_size][row].
struct CacheStrides {
  int64_t block;  // between blocks
  int tok;        // between the rows of consecutive tokens of one head
  int head;       // between the rows of consecutive heads of one token
};
__host__ __device__ inline CacheStrides cache_strides(uint32_t flags, int block_size, int num_kv_heads, int row) {
  const int64_t block = (int64_t)block_size * num_kv_heads * row;
  return (flags & LGM_CACHE_HND) ? CacheStrides{block, row, block_size * row}
                                 : CacheStrides{block, num_kv_heads * row, row};
}
// The FP8 scale of kv head g: per head, or the one per-tensor value.
__host__ __device__ inline float kv_scale(const float* s, uint32_t flags, int g) {
  return s[(flags & LGM_SCALE_PER_TENSOR) ? 0 : g];
}

struct MergeArgs {
  void* out;
  float* out_lse;
  const float* part_out;
  const float* part_lse;
  const int32_t* num_partitions;  // per sequence, or NULL
  const int32_t* context_lens;    // alternative source of the count (parts.count)
  PartitionPlan parts;
  int32_t max_context_len;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t max_partitions;
  int32_t skip_single;            // 1: sequences with <= 1 partition were written directly
};

// Each returns hipSuccess or the launch error.
hipError_t launch_rope_kv_append(const AppendArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s);
// Read-only streaming probe: bytes must be a multiple of num_wg *
// stream_probe_granule(), and bytes / num_wg must fit in an int.
int stream_probe_granule();
hipError_t launch_stream_read_probe(const void* src, int64_t bytes, int num_wg, bool nontemporal, uint32_t* sink,
                                    hipStream_t s);
hipError_t launch_paged_decode(const DecodeArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, lgm_dtype out_dtype, hipStream_t s);
hipError_t launch_table_check(const int32_t* block_tables, const int32_t* context_lens, const lgm_paged_dims& d,
                              int32_t max_context_len, int32_t* status, hipStream_t s);

// Matrix-core decode for bf16 activations with bf16 / FP8 caches, head_dim 128.
hipError_t launch_paged_decode_mfma(const DecodeArgs& a, lgm_dtype cache, hipStream_t s);
// Whole-row decode (matrix-core shapes): equal static tile ranges, one per
// workgroup, then a merge of the split streams.
// Head groups of 8 kv heads only up to this many query heads per kv head
// (the planner's rule; the kernel builds no 8-head shape past it).
#ifndef LGM_ROWS_HG8_MAX_GROUP
#define LGM_ROWS_HG8_MAX_GROUP 8
#endif
struct RowsArgs {
  int32_t num_wg;         // W: workgroups, one range each
  int32_t head_group;     // HG: kv heads per workgroup (8 or 4; 2 or 1 with 2 or 4 token slices per head)
  float* rec_out;         // [W][2][HG * G][D] normalised partial outputs
  float* rec_lse;         // [W][2][HG * G] natural-log LSEs
  int32_t* wg_first;  // [B * Hkv / HG] record slot of the stream's first piece (2w or 2w + 1 for range w)
  int32_t* wg_last;   // [B * Hkv / HG] workgroup holding its last tile
  // > 0: the ranges are cut into split-K partitions of this many 32-token
  // tiles instead (whole partitions per workgroup); each partition's record
  // goes to DecodeArgs::part_out / part_lse and lse_merge combines them.
  int32_t part_tiles;
};
hipError_t launch_paged_decode_rows(const DecodeArgs& a, const RowsArgs& r, lgm_dtype cache, hipStream_t s);
bool decode_rows_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int num_kv_heads, int group,
                           int block_size);

// Single-launch split-K decode for small jobs (matrix-core shapes): one
// workgroup per (sequence, kv head, partition), the last workgroup to finish
// one of a context's partitions merges its records.  The arrival counters
// sit in the workspace's counter slot, after the work-queue kernel's two.
constexpr int kFusedMaxChunks = 64;   // partitions per context
constexpr int kFusedMaxStreams = (int)(LGM_COUNTER_SLOT_BYTES / 4) - 2;  // arrival counters: slot words 2 ..
struct FusedArgs {
  int32_t chunk_steps;  // a partition is 4 waves x chunk_steps x 32 tokens (chunk_steps <= 32)
  int32_t nchunks;      // partitions per context at max_context_len; grid B * Hkv * nchunks
  float* rec_out;       // [B * Hkv][nchunks][G][D] normalised partial outputs
  float* rec_lse;       // [B * Hkv][nchunks][G] natural-log LSEs
  int32_t rec_out_bytes, rec_lse_bytes;
  int32_t* arrivals;    // [B * Hkv] zero on entry, left zero on completion
};
hipError_t launch_paged_decode_fused(const DecodeArgs& a, const FusedArgs& f, lgm_dtype cache, hipStream_t s);

// Upper bound on the persistent matrix-core kernel's workgroups per compute
// unit (the grid is compute units x min(this, resident capacity)).
#ifndef LGM_PERSISTENT_MAX_PER_CU
#define LGM_PERSISTENT_MAX_PER_CU 2
#endif
constexpr int kPersistentMaxPerCU = LGM_PERSISTENT_MAX_PER_CU;

// Paged MLA decode: one workgroup per (sequence, partition), grid
// (max_partitions, num_seqs).
struct MlaArgs {
  void* out;                // [B][H][512] bf16
  float* out_lse;           // [B][H] or NULL
  const void* q_latent;     // [B][H][512] bf16
  const void* q_pe;         // [B][H][64] bf16
  const void* ckv;          // [NB][bs][512] FP8 codes
  const void* kpe;          // [NB][bs][64] bf16
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* ckv_scale;   // [1]
  float* part_out;          // [B][H][P][512] fp32, NULL when P == 1
  float* part_lse;          // [B][H][P]
  float softmax_scale;
  int32_t partition_size;   // multiple of 32
  int32_t max_context_len;
  int32_t max_partitions;   // P
  lgm_mla_dims dims;
};
hipError_t launch_paged_mla(const MlaArgs& a, hipStream_t s);
bool mla_supported(lgm_dtype ckv, int latent_dim, int rope_dim, int num_heads, int block_size);

// Shape support queries used by validation (no HIP calls).
bool decode_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool decode_valu_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool decode_mfma_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool merge_supported(int head_dim);

}  // namespace lgm
