// Internal interface between the C-ABI host layer (lgm_api.cpp) and the
// kernel translation units.  Arguments reaching a launcher have already been
// validated by the host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lgm.h"

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
  float softmax_scale;
  int32_t partition_size;
  int32_t max_context_len;
  int32_t max_partitions;
  lgm_paged_dims dims;
};

struct MergeArgs {
  void* out;
  float* out_lse;
  const float* part_out;
  const float* part_lse;
  const int32_t* num_partitions;  // per sequence, or NULL
  const int32_t* context_lens;    // alternative source of the count (with partition_size)
  int32_t partition_size;
  int32_t max_context_len;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t max_partitions;
  int32_t skip_single;            // 1: sequences with <= 1 partition were written directly
};

// Each returns hipSuccess or the launch error.
hipError_t launch_rope_kv_append(const AppendArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s);
hipError_t launch_paged_decode(const DecodeArgs& a, lgm_dtype act, lgm_dtype cache, hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, lgm_dtype out_dtype, hipStream_t s);

// Shape support queries used by validation (no HIP calls).
bool decode_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool merge_supported(int head_dim);

}  // namespace lgm
