// Opt-in check of the device-resident block tables and context lengths, the
// span check the mainarch README's troubleshooting section describes for its
// VA guard, here for the paged-KV contract.  The decode and append kernels
// mask an out-of-range table entry inside a context (its 16 tokens are left
// out, the append's write is skipped) and clamp context lengths, silently;
// this kernel reads the same entries with the same clamping and reports what
// those kernels would mask, into caller-provided device words.
#include "lgm_internal.h"

namespace lgm {
namespace {

constexpr int kCheckThreads = 256;

// One workgroup per sequence.  status (zero before the first check):
//   [0] += table entries inside a context outside [0, num_blocks)
//   [1] += sequences whose context_lens exceeds max_blocks_per_seq *
//          block_size or max_context_len (the kernels clamp it)
//   [2]  = max over bad entries of 0x7FFFFFFF - (b * max_blocks_per_seq + lb),
//          so the first bad (sequence, logical block) is 0x7FFFFFFF - [2]
__global__ __launch_bounds__(kCheckThreads) void table_check_kernel(const int32_t* block_tables,
                                                                   const int32_t* context_lens, lgm_paged_dims d,
                                                                   int32_t max_context_len, int32_t* status) {
  const int b = blockIdx.x;
  const int MB = d.max_blocks_per_seq;
  const int64_t cap = (int64_t)MB * d.block_size;
  const int raw = context_lens[b];
  int ctx = raw < 0 ? 0 : raw;
  if (threadIdx.x == 0 && (ctx > cap || ctx > max_context_len)) atomicAdd(status + 1, 1);
  ctx = (int)(ctx > cap ? cap : ctx);
  const int used = (ctx + d.block_size - 1) / d.block_size;
  const int32_t* row = block_tables + (int64_t)b * MB;
  int bad = 0, first = -1;
  for (int lb = threadIdx.x; lb < used; lb += kCheckThreads) {
    const int id = row[lb];
    if ((unsigned)id >= (unsigned)d.num_blocks) {
      ++bad;
      if (first < 0) first = lb;
    }
  }
  if (bad) {
    atomicAdd(status, bad);
    atomicMax(status + 2, (int)(0x7FFFFFFF - ((int64_t)b * MB + first)));
  }
}

}  // namespace

hipError_t launch_table_check(const int32_t* block_tables, const int32_t* context_lens, const lgm_paged_dims& d,
                              int32_t max_context_len, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(table_check_kernel, dim3(d.num_seqs), dim3(kCheckThreads), 0, s, block_tables, context_lens, d,
                     max_context_len, status);
  return hipGetLastError();
}

}  // namespace lgm
