// Log-sum-exp merge of split-K partition records (mainarch README,
// decode-attention section: split partials are combined in parallel rather
// than by one workgroup grinding through them; Loom Kernels README, row
// "Attention": local split-K/LSE merge).
//
// One workgroup per (sequence, head) or, when there are few rows (long
// contexts, many partitions each), per (sequence, head, 32-element slice of
// the head dim), so that a row's partitions are read by D/32 workgroups side
// by side.  Each reduces the partition LSEs to their maximum M and to
// S = sum exp(lse_p - M) with fixed-shape tree reductions in LDS; its slice
// of the partial rows is then read with 16-byte loads, 256 / (SL/4) records
// at a time, weighted by exp(lse_p - M) and summed, and the partial sums are
// added in a fixed order.  The result is bitwise reproducible.
#include "device_num.h"
#include "lgm_internal.h"

namespace lgm {
namespace {

constexpr int kThreads = 256;

struct OutF32 {
  using elem_t = float;
  __device__ static elem_t from_f32(float x) { return x; }
};
struct OutBF16 {
  using elem_t = uint16_t;
  __device__ static elem_t from_f32(float x) { return f32_to_bf16_rne(x); }
};

template <bool kMax>
__device__ float block_reduce(float x, float* red) {
  red[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const float a = red[threadIdx.x], c = red[threadIdx.x + s];
      red[threadIdx.x] = kMax ? fmaxf(a, c) : a + c;
    }
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

constexpr int kNarrowSlice = 32;     // head-dim elements per workgroup when rows are few
constexpr int64_t kFewRows = 1024;   // below this many (sequence, head) rows, slice the head dim

template <class O, int D, int SL>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(MergeArgs p) {
  constexpr int TD = SL / 4;         // lanes per record slice (float4 each)
  constexpr int PG = kThreads / TD;  // records in flight per pass
  __shared__ float red[kThreads];
  __shared__ float s_acc[PG][SL];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int z = blockIdx.z;  // which slice of the head dim
  const int P = p.max_partitions;
  int n;
  if (p.num_partitions) {
    n = p.num_partitions[b];
    n = n < 0 ? 0 : (n > P ? P : n);
  } else if (p.context_lens) {
    int ctx = p.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
    n = p.parts.count(ctx);
    n = n > P ? P : n;
  } else {
    n = P;
  }
  if (p.skip_single && n <= 1) return;

  const int64_t row = (int64_t)b * p.num_heads + h;
  const float* lse = p.part_lse + row * P;
  const float* po = p.part_out + row * P * D + z * SL;

  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kThreads) mx = fmaxf(mx, lse[i]);
  const float M = block_reduce<true>(mx, red);
  const float ms = M == -INFINITY ? 0.f : M;
  float sw = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) sw += expf(lse[i] - ms);
  const float S = block_reduce<false>(sw, red);

  const int td = threadIdx.x % TD;
  const int pg = threadIdx.x / TD;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int i = pg; i < n; i += PG) {
    // A record of weight zero (lse = -inf: an empty partition) is left out
    // by a select, so its row may hold anything, NaN included.
    const float w = expf(lse[i] - ms);
    const float4 v = reinterpret_cast<const float4*>(po + (int64_t)i * D)[td];
    const bool live = w != 0.f;
    a.x = live ? fmaf(w, v.x, a.x) : a.x;
    a.y = live ? fmaf(w, v.y, a.y) : a.y;
    a.z = live ? fmaf(w, v.z, a.z) : a.z;
    a.w = live ? fmaf(w, v.w, a.w) : a.w;
  }
  s_acc[pg][td * 4 + 0] = a.x;
  s_acc[pg][td * 4 + 1] = a.y;
  s_acc[pg][td * 4 + 2] = a.z;
  s_acc[pg][td * 4 + 3] = a.w;
  __syncthreads();
  for (int d = threadIdx.x; d < SL; d += kThreads) {
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < PG; ++k) o += s_acc[k][d];
    o = S > 0.f ? o / S : 0.f;
    static_cast<typename O::elem_t*>(p.out)[row * D + z * SL + d] = O::from_f32(o);
  }
  if (z == 0 && threadIdx.x == 0 && p.out_lse) p.out_lse[row] = S > 0.f ? M + logf(S) : -INFINITY;
}

template <class O, int D>
void launch_dim(const MergeArgs& a, hipStream_t s) {
  if ((int64_t)a.num_seqs * a.num_heads < kFewRows)
    hipLaunchKernelGGL((lse_merge_kernel<O, D, kNarrowSlice>), dim3(a.num_heads, a.num_seqs, D / kNarrowSlice),
                       dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<O, D, D>), dim3(a.num_heads, a.num_seqs, 1), dim3(kThreads), 0, s, a);
}

template <class O>
hipError_t dispatch(const MergeArgs& a, hipStream_t s) {
  if (a.head_dim == 64)
    launch_dim<O, 64>(a, s);
  else if (a.head_dim == 128)
    launch_dim<O, 128>(a, s);
  else if (a.head_dim == 512)  // the MLA latent
    launch_dim<O, 512>(a, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool merge_supported(int head_dim) { return head_dim == 64 || head_dim == 128 || head_dim == 512; }

hipError_t launch_lse_merge(const MergeArgs& a, lgm_dtype out_dtype, hipStream_t s) {
  if (out_dtype == LGM_F32) return dispatch<OutF32>(a, s);
  if (out_dtype == LGM_BF16) return dispatch<OutBF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace lgm
