// Scalar split kernel: one 64-lane wavefront per (query row, split), fp32 FMA.
//
// It serves the fp32 dtype and is the plain, easy-to-audit path for bf16. Each
// wavefront walks its split's key range one key at a time ("The Architecture of
// Capture Safety", "The Design Emerges", first insight: split s covers
// [s*chunk, min((s+1)*chunk, N)) with chunk = ceil(N / nsplit), and an empty
// split returns at once), resolves the key's cache slot from kv_indices
// (prefix) or out_cache_loc (draft tokens) (second insight), reads the
// visibility byte from custom_mask at mask_indptr[b] + i*N + p (third insight),
// and keeps an online softmax: running max m, running sum l and a rescaled
// output accumulator o ("The Architecture of Capture Safety", "Input Knowledge
// Required").
//
// Lane l owns latent entries [8l, 8l+8) and rope entry l of the 576-wide
// key, so one cache row is read as 64 contiguous 16-byte pieces plus one
// 128-byte rope segment; the dot product is a wavefront butterfly sum.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bits
  __device__ static void load8(const uint16_t* p, float* v) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  __device__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store8(uint16_t* p, const float* v) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
  }
};

template <>
struct Elem<float> {
  __device__ static void load8(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static float load1(const float* p) { return *p; }
};

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T>
__global__ __launch_bounds__(256) void split_scalar_kernel(SplitParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int Rw = p.num_draft * p.num_heads;  // partial-row stride of the workspace
  const int r = blockIdx.x * 4 + wave;
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  int Tb;
  int64_t tb;  // draft tokens of request b, and the first one
  request_tokens(p.qo_indptr, p.num_draft, b, Tb, tb);
  if (r >= Tb * p.num_heads) return;

  const int ip0 = p.kv_indptr[b];
  const int P = p.kv_indptr[b + 1] - ip0;
  const int N = P + Tb;
  int start, end;
  split_bounds(N, p.nsplit, p.min_chunk, p.chunk_align, s, start, end);
  if (start >= end) return;  // empty split: nothing to write, the combine skips it

  const int i = r / p.num_heads;
  const int h = r - i * p.num_heads;
  const int64_t t = tb + i;

  const T* qn = static_cast<const T*>(p.q_nope) + t * p.qn_stride_tok + h * p.qn_stride_head;
  const T* qr = static_cast<const T*>(p.q_rope) + t * p.qr_stride_tok + h * p.qr_stride_head;
  float q[8];
  Elem<T>::load8(qn + 8 * lane, q);
  const float q_r = Elem<T>::load1(qr + lane);

  const float scale2 = p.sm_scale * kLog2e;  // scores kept in log2 units
  const uint8_t* mrow = p.mask + p.mask_indptr[b] + (int64_t)i * N;
  const T* kv = static_cast<const T*>(p.kv);

  float m = -INFINITY, l = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = start; k < end; ++k) {
    if (mrow[k] == 0) continue;  // wave-uniform branch
    const int slot = k < P ? p.kv_indices[ip0 + k] : p.out_cache_loc[t - i + (k - P)];
    const T* row = kv + (int64_t)slot * p.kv_stride;
    float v[8];
    Elem<T>::load8(row + 8 * lane, v);
    const float kr = Elem<T>::load1(row + kDLatent + lane);
    float d = q_r * kr;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(q[e], v[e], d);
    const float sc = wave_sum(d) * scale2;
    const float mn = fmaxf(m, sc);
    const float alpha = exp2f(m - mn);  // m = -inf on the first visible key -> 0
    const float beta = exp2f(sc - mn);
    l = l * alpha + beta;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(beta, v[e], o[e] * alpha);
    m = mn;
  }

  const size_t prow = ((size_t)b * p.nsplit + s) * Rw + r;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (sizeof(T) == 2) {  // bf16 queries: the row as bf16 in the slot's first 1 KB
    uint16_t* dst = partial_bf16(p.o_part, prow) + 8 * lane;
    const uint2 a = pack_bf16x4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    const uint2 c = pack_bf16x4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, c.x, c.y);
  } else {
    float* dst = p.o_part + prow * kDLatent + 8 * lane;
    float4 a, c;
    a.x = o[0] * inv; a.y = o[1] * inv; a.z = o[2] * inv; a.w = o[3] * inv;
    c.x = o[4] * inv; c.y = o[5] * inv; c.z = o[6] * inv; c.w = o[7] * inv;
    reinterpret_cast<float4*>(dst)[0] = a;
    reinterpret_cast<float4*>(dst)[1] = c;
  }
  if (lane == 0) p.lse_part[prow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <typename T>
hipError_t launch(const SplitParams& p, hipStream_t stream) {
  const int R = p.num_draft * p.num_heads;
  dim3 grid((R + 3) / 4, p.nsplit, p.batch);
  SplitParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&split_scalar_kernel<T>), grid, dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_split_scalar_bf16(const SplitParams& p, hipStream_t stream) { return launch<uint16_t>(p, stream); }
hipError_t launch_split_scalar_fp32(const SplitParams& p, hipStream_t stream) { return launch<float>(p, stream); }

}  // namespace tvmla
