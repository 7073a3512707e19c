// Matrix-core throughput probe for gfx950: the dense bf16 MFMA rate this part
// sustains, measured beside the split kernel so its MFMA fraction can be read
// against the hardware as well as against the published peak. Not part of
// the verify path: bench.py compiles it (build_probe) into
// libtvmla_probe.so beside itself and loads it from there.
//
// Every wavefront runs `iters` rounds of eight independent accumulation
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

}  // namespace

extern "C" {

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
