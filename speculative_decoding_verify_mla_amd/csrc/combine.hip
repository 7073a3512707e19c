// Combine kernel: log-sum-exp merge of the per-split partial results.
//
// The reduce step of the split-K flash-decode ("The Architecture of Capture
// Safety", "The Design Emerges", first insight). Split s left o_s (its output,
// normalised by its own softmax sum) and lse_s (natural log of that sum); the
// merged row is
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + log(sum_s w_s).
// Splits that hold no keys under the schedule never wrote anything and are
// not read, so the workspace needs no clearing between calls; a split that
// held keys but saw none of them wrote lse_s = -inf and weighs nothing.
//
// W wavefronts per output row, W in {1, 4, 16}, chosen from the row count so
// that a launch has enough wavefronts in flight to keep HBM busy. Wavefront w
// of the row takes splits s = w, w+W, w+2W, ...: the row's split maximum and
// weight sum are reductions over their lse_s, and the wavefront accumulates
// their weighted partial rows (lane l owns entries [8l, 8l+8); four to
// sixteen partial rows in flight per wavefront); for W > 1 the accumulators
// are added through LDS. A partial row is 1 KB of bf16 (bf16
// queries) or 2 KB of fp32 (fp32 queries), read contiguously (HBM-bound).

#include "tvmla.h"
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


// W wavefronts per row; a workgroup holds kRowsWG = max(1, 4 / W) rows.
// Wavefront wr of a row takes the row's splits s = wr + W*u (u = 0, 1, ...).
// It reads their lse_s and, without waiting for them, the first kUnroll of
// their partial rows; the row maximum comes from a wavefront maximum (and,
// for W > 1, an exchange through LDS); each lane turns its splits' lse_s
// into weights, which go to a per-wavefront LDS table the accumulation loop
// reads back (no barrier: the same wavefront writes and reads it, and its
// LDS operations complete in order). One memory round trip before the
// first accumulation instead of three dependent ones.
template <bool kBf16, int W>
__global__ __launch_bounds__(W == 16 ? 1024 : 256) void combine_kernel(CombineParams c) {
  constexpr int kRowsWG = W >= 4 ? 1 : 4 / W;
  constexpr int kWaves = kRowsWG * W;
  // partial rows in flight per wavefront (bf16 rows are half the bytes: twice as many)
  constexpr int kUnroll = (W == 1 ? 4 : 8) * (kBf16 ? 2 : 1);
  constexpr int kPerWave = (TVMLA_MAX_NSPLIT + W - 1) / W;  // splits one wavefront may hold
  constexpr int kPerLane = (kPerWave + 63) / 64;
  __shared__ float red_m[kWaves], red_l[kWaves];
  __shared__ float wtab[kWaves][kPerWave];
  __shared__ __attribute__((aligned(16))) float red_o[W > 1 ? W - 1 : 1][kDLatent];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wr = wave % W;  // wavefront within its row
  const int R = c.num_draft * c.num_heads;
  const int64_t row = (int64_t)blockIdx.x * kRowsWG + wave / W;
  if (row >= (int64_t)c.batch * R) return;  // only with W = 1; no barrier follows then
  const int b = (int)(row / R);
  const int r = (int)(row - (int64_t)b * R);
  int Tb;
  int64_t tb;  // draft tokens of request b, and the first one
  request_tokens(c.qo_indptr, c.num_draft, b, Tb, tb);
  if (r >= Tb * c.num_heads) return;  // one row per workgroup when W > 1: no barrier is left behind
  const int64_t orow = tb * c.num_heads + r;  // output row
  int ns = c.nsplit;
  if (c.kv_indptr != nullptr) {
    const int n = c.kv_indptr[b + 1] - c.kv_indptr[b] + Tb;
    ns = active_splits(n, c.nsplit, c.min_chunk, c.chunk_align);
  }
  const size_t base = (size_t)b * c.nsplit * R + r;  // partial row of split 0
  const int nu = ns > wr ? (ns - wr + W - 1) / W : 0;  // this wavefront's splits

  // one partial row's 8 entries of this lane: [8 lane, 8 lane + 8)
  auto load_row = [&](int u) -> uint4 {
    const size_t pr = base + (size_t)(wr + W * u) * R;
    if (kBf16)  // bf16 partial rows: the slot's first 1 KB
      return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(c.o_part + pr * kDLatent) + 8 * lane);
    return uint4{};
  };
  auto load_row32 = [&](int u, float4& a, float4& d) {
    const size_t pr = base + (size_t)(wr + W * u) * R;
    const float4* src = reinterpret_cast<const float4*>(c.o_part + pr * kDLatent + 8 * lane);
    a = src[0];
    d = src[1];
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto fma_row = [&](float w, float4 a, float4 d) {
    if (w > 0.f) {  // a split whose row saw no visible key (lse_s = -inf) weighs nothing
      acc[0] = fmaf(w, a.x, acc[0]); acc[1] = fmaf(w, a.y, acc[1]);
      acc[2] = fmaf(w, a.z, acc[2]); acc[3] = fmaf(w, a.w, acc[3]);
      acc[4] = fmaf(w, d.x, acc[4]); acc[5] = fmaf(w, d.y, acc[5]);
      acc[6] = fmaf(w, d.z, acc[6]); acc[7] = fmaf(w, d.w, acc[7]);
    }
  };
  auto unpack = [](uint4 u, float4& a, float4& d) {
    a = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                    __uint_as_float(u.y & 0xffff0000u));
    d = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u), __uint_as_float(u.w << 16),
                    __uint_as_float(u.w & 0xffff0000u));
  };

  // the first batch of partial rows, in flight while the weights are formed
  uint4 pre16[kBf16 ? kUnroll : 1];
  float4 pre32a[kBf16 ? 1 : kUnroll], pre32d[kBf16 ? 1 : kUnroll];
  const int npre = nu < kUnroll ? nu : kUnroll;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (u < npre) {
      if (kBf16)
        pre16[kBf16 ? u : 0] = load_row(u);
      else
        load_row32(u, pre32a[kBf16 ? 0 : u], pre32d[kBf16 ? 0 : u]);
    }
  }

  // row maximum of lse_s
  float lv[kPerLane];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int u = lane + 64 * j;
    lv[j] = u < nu ? c.lse_part[base + (size_t)(wr + W * u) * R] : -INFINITY;
    mx = fmaxf(mx, lv[j]);
  }
  mx = wave_max(mx);
  if (W > 1) {
    if (lane == 0) red_m[wave] = mx;
    __syncthreads();
    mx = red_m[0];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, red_m[w]);
  }
  // weights, their sum, and the table the accumulation reads
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int u = lane + 64 * j;
    const float w = mx != -INFINITY && lv[j] != -INFINITY ? exp2f((lv[j] - mx) * kLog2e) : 0.f;
    wsum += w;
    if (u < kPerWave) wtab[wave][u] = w;
  }
  wsum = wave_sum(wsum);

#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (u < npre) {
      float4 a, d;
      if (kBf16)
        unpack(pre16[kBf16 ? u : 0], a, d);
      else
        a = pre32a[kBf16 ? 0 : u], d = pre32d[kBf16 ? 0 : u];
      fma_row(wtab[wave][u], a, d);
    }
  }
  for (int u0 = kUnroll; u0 < nu; u0 += kUnroll) {
    uint4 raw16[kBf16 ? kUnroll : 1];
    float4 ra[kBf16 ? 1 : kUnroll], rd[kBf16 ? 1 : kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u0 + u < nu) {
        if (kBf16)
          raw16[kBf16 ? u : 0] = load_row(u0 + u);
        else
          load_row32(u0 + u, ra[kBf16 ? 0 : u], rd[kBf16 ? 0 : u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u0 + u < nu) {
        float4 a, d;
        if (kBf16)
          unpack(raw16[kBf16 ? u : 0], a, d);
        else
          a = ra[kBf16 ? 0 : u], d = rd[kBf16 ? 0 : u];
        fma_row(wtab[wave][u0 + u], a, d);
      }
    }
  }
  if (W > 1) {
    if (lane == 0) red_l[wave] = wsum;
    if (wr > 0) {
      float4* dst = reinterpret_cast<float4*>(&red_o[wr - 1][8 * lane]);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wr != 0) return;
    wsum = red_l[0];
#pragma unroll
    for (int w = 1; w < W; ++w) wsum += red_l[w];
#pragma unroll
    for (int w = 0; w < W - 1; ++w) {
      const float4* src = reinterpret_cast<const float4*>(&red_o[w][8 * lane]);
      const float4 a = src[0], d = src[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += d.x; acc[5] += d.y; acc[6] += d.z; acc[7] += d.w;
    }
  }
  if (mx != -INFINITY) {
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }

  if (kBf16) {
    uint16_t* dst = static_cast<uint16_t*>(c.out) + orow * kDLatent + 8 * lane;
    uint4 u;
    u.x = pack_bf16x2(acc[0], acc[1]);
    u.y = pack_bf16x2(acc[2], acc[3]);
    u.z = pack_bf16x2(acc[4], acc[5]);
    u.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(dst) = u;
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(c.out) + orow * kDLatent + 8 * lane);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (lane == 0) c.lse[orow] = mx != -INFINITY ? mx + logf(wsum) : -INFINITY;
}

template <int W>
hipError_t launch_w(const CombineParams& c, int dtype, int64_t rows, hipStream_t stream) {
  constexpr int kRowsWG = W >= 4 ? 1 : 4 / W;
  dim3 grid((unsigned)((rows + kRowsWG - 1) / kRowsWG));
  CombineParams arg = c;
  void* args[] = {&arg};
  const void* fn = dtype == 0 ? reinterpret_cast<const void*>(&combine_kernel<true, W>)
                              : reinterpret_cast<const void*>(&combine_kernel<false, W>);
  return hipLaunchKernel(fn, grid, dim3(W == 16 ? 1024 : 256), args, 0, stream);
}

}  // namespace

hipError_t launch_combine(const CombineParams& c, int dtype, hipStream_t stream) {
  // enough wavefronts for HBM: ~4096 rows and up take one each, fewer rows more
  const int64_t rows = (int64_t)c.batch * c.num_draft * c.num_heads;
  if (rows >= 4096) return launch_w<1>(c, dtype, rows, stream);
  if (rows >= 512) return launch_w<4>(c, dtype, rows, stream);
  return launch_w<16>(c, dtype, rows, stream);
}

}  // namespace tvmla
