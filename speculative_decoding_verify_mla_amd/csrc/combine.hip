// Combine kernel: log-sum-exp merge of the per-split partial results.
//
// The reduce step of the split-K flash-decode (page 1, "The Design Emerges",
// first insight). Split s left o_s (its output, normalised by its own
// softmax sum) and lse_s (natural log of that sum); the merged row is
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + log(sum_s w_s).
// Splits that hold no keys under the schedule never wrote anything and are
// not read, so the workspace needs no clearing between calls; a split that
// held keys but saw none of them wrote lse_s = -inf and weighs nothing.
//
// One 64-lane wavefront per output row; lane l owns entries [8l, 8l+8).
// The partial rows are read as 2 KB contiguous segments (HBM-bound).

#include "tvmla_internal.h"

namespace tvmla {
namespace {

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams c) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int R = c.num_draft * c.num_heads;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= (int64_t)c.batch * R) return;
  const int b = (int)(row / R);
  const int r = (int)(row - (int64_t)b * R);

  int ns = c.nsplit;
  if (c.kv_indptr != nullptr) {
    const int n = c.kv_indptr[b + 1] - c.kv_indptr[b] + c.num_draft;
    ns = active_splits(n, c.nsplit, c.min_chunk);
  }
  const size_t base = (size_t)b * c.nsplit * R + r;  // partial row of split 0

  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, c.lse_part[base + (size_t)s * R]);
  mx = wave_max(mx);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = lane; s < ns; s += 64) wsum += exp2f((c.lse_part[base + (size_t)s * R] - mx) * kLog2e);
    wsum = wave_sum(wsum);
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const size_t pr = base + (size_t)s * R;
      const float w = exp2f((c.lse_part[pr] - mx) * kLog2e);
      const float4* src = reinterpret_cast<const float4*>(c.o_part + pr * kDLatent + 8 * lane);
      const float4 a = src[0], d = src[1];
      if (w > 0.f) {
        acc[0] = fmaf(w, a.x, acc[0]); acc[1] = fmaf(w, a.y, acc[1]);
        acc[2] = fmaf(w, a.z, acc[2]); acc[3] = fmaf(w, a.w, acc[3]);
        acc[4] = fmaf(w, d.x, acc[4]); acc[5] = fmaf(w, d.y, acc[5]);
        acc[6] = fmaf(w, d.z, acc[6]); acc[7] = fmaf(w, d.w, acc[7]);
      }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }

  if (kBf16) {
    uint16_t* dst = static_cast<uint16_t*>(c.out) + row * kDLatent + 8 * lane;
    uint4 u;
    u.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    u.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    u.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(dst) = u;
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(c.out) + row * kDLatent + 8 * lane);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (lane == 0) c.lse[row] = mx != -INFINITY ? mx + logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams& c, int dtype, hipStream_t stream) {
  const int64_t rows = (int64_t)c.batch * c.num_draft * c.num_heads;
  dim3 grid((unsigned)((rows + 3) / 4));
  CombineParams arg = c;
  void* args[] = {&arg};
  const void* fn = dtype == 0 ? reinterpret_cast<const void*>(&combine_kernel<true>)
                              : reinterpret_cast<const void*>(&combine_kernel<false>);
  return hipLaunchKernel(fn, grid, dim3(256), args, 0, stream);
}

}  // namespace tvmla
