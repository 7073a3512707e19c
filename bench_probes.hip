// Throughput probes for gfx950, measured beside the verify call so its
// roofline fractions can be read against what this part sustains as well as
// against the published peaks. Not part of the verify path: bench.py
// compiles them (build_probe) into libtvmla_probe.so beside itself and loads
// them from there.
//
// MFMA probe: the dense bf16 MFMA rate. Every wavefront runs `iters` rounds of eight independent accumulation
// chains of v_mfma_f32_32x32x16_bf16 (32x32 outputs, k = 16: 32,768 flops
// each) on register operands, two workgroups of four wavefronts per compute
// unit, so each SIMD always has an independent MFMA ready to issue. The sum
// of the accumulators goes to `sink` (one float per thread) so the work is
// kept.

#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  f32x16_t acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Read probes. stream_read_kernel: a grid-stride read of n16 16-byte words
// (a running xor keeps the loads). gather_rows_kernel: the verify path's
// access pattern without its arithmetic -- each wavefront takes units of 8
// cache rows of row_bytes (a multiple of 16, at most 2,304) from the slots
// list, lanes 0..7 read the 8 slots, and the rows' 16-byte pieces are spread
// over the 64 lanes with every load of a unit issued before any is used.
// Both load non-temporally, as the verify kernels stage the cache rows: a
// cold read that allocates in a MALL full of other dirty lines also pays
// for their write-back.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t n16, unsigned* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    acc ^= __builtin_nontemporal_load(src + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

constexpr int kMaxPieces = 2304 / 16;  // 16-byte pieces of the largest row (fp32, 576 entries)

__global__ __launch_bounds__(256) void gather_rows_kernel(const char* pool, long row_bytes, const int* slots,
                                                          int nrows, unsigned* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pieces = (int)(row_bytes / 16);
  const int per_lane = (8 * pieces + 63) / 64;  // at most 18
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int u = blockIdx.x * 4 + wave; 8 * u < nrows; u += gridDim.x * 4) {
    const int nr = nrows - 8 * u < 8 ? nrows - 8 * u : 8;
    const long slot = lane < nr ? (long)slots[8 * u + lane] : 0;
    u32x4 v[(8 * kMaxPieces + 63) / 64];
#pragma unroll
    for (int k = 0; k < (8 * kMaxPieces + 63) / 64; ++k) {
      v[k] = u32x4{0u, 0u, 0u, 0u};
      const int id = lane + 64 * k, r = id / pieces, c = id - r * pieces;
      const long s = __shfl(slot, r < nr ? r : nr - 1, 64);
      if (k < per_lane && r < nr)
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pool + s * row_bytes + 16 * c));
    }
#pragma unroll
    for (int k = 0; k < (8 * kMaxPieces + 63) / 64; ++k) acc ^= v[k];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

}  // namespace

extern "C" {

// A streaming read of `bytes` (a multiple of 16) from src; `sink` >= 4 bytes
// of device memory. Returns the HIP status of the launch.
int tvmla_probe_stream_read(const void* src, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (src == nullptr || sink == nullptr || blocks <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

// A gather of nrows rows of row_bytes (16 <= row_bytes <= 2304, a multiple
// of 16) at pool + slots[i] * row_bytes. Returns the HIP status of the
// launch.
int tvmla_probe_gather_rows(const void* pool, long row_bytes, const int* slots, int nrows, unsigned* sink, int blocks,
                            void* stream) {
  if (pool == nullptr || slots == nullptr || sink == nullptr || blocks <= 0 || nrows < 0 || row_bytes < 16 ||
      row_bytes > 2304 || row_bytes % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const char*>(pool), row_bytes, slots, nrows, sink);
  return (int)hipGetLastError();
}


// Flops one launch performs: blocks x 4 wavefronts x iters x 8 chains x
// 32,768. `sink` holds blocks * 256 floats (device memory). Returns the HIP
// status of the launch (0 = success).
double tvmla_probe_mfma_flops(int blocks, int iters) { return (double)blocks * 4.0 * iters * kChains * 32768.0; }

int tvmla_probe_mfma_bf16(float* sink, int blocks, int iters, void* stream) {
  if (sink == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
