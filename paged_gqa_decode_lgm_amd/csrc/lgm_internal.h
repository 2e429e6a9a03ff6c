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

// Balanced decode: records of split segments and their arrival counts.
struct StreamArgs {
  int32_t num_waves;       // W: the tiles of all segments are cut into W equal ranges
  int32_t record_floats;   // floats per record (stream_record_floats(G))
  float* records;          // [W][2][record_floats]
  int32_t* counters;       // [B][Hkv], zero on entry, left zero on completion
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

// Matrix-core decode for bf16 activations with bf16 / FP8 caches, head_dim 128.
hipError_t launch_paged_decode_mfma(const DecodeArgs& a, lgm_dtype cache, hipStream_t s);
// The same shapes with balanced tile ranges, one launch (partition_size 0).
hipError_t launch_paged_decode_stream(const DecodeArgs& a, const StreamArgs& x, lgm_dtype cache, hipStream_t s);
int stream_record_floats(int group);

// Minimum resident waves per SIMD the balanced kernel is compiled for; the
// host cuts the work into (compute units x 4 x this) ranges so that all of
// them run at once.
constexpr int stream_waves_per_simd(bool fp8_cache, int group) { return fp8_cache ? 3 : (group <= 4 ? 3 : 2); }

// Shape support queries used by validation (no HIP calls).
bool decode_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool decode_valu_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool decode_mfma_supported(lgm_dtype act, lgm_dtype cache, int head_dim, int group, int block_size);
bool merge_supported(int head_dim);

}  // namespace lgm
