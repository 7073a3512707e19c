// Visibility mask of a draft tree, built on the device from parent arrays.
//
// A DDTree drafter proposes a tree of draft tokens that the target model
// verifies in one pass, and the verify attention needs a mask of which draft
// token sees which key ("The Architecture of Capture Safety: Designing a CUDA
// Graph-Compatible Verify Kernel for SGLang", section "Input Knowledge
// Required", DDTree paragraph), passed raw as custom_mask + mask_indptr (same
// page, section "The Design Emerges", third insight). Building it here keeps
// that marshaling on the GPU and inside a captured graph.
//
// Row i of request b (P_b prefix keys, N_b = P_b + T) is 1 on every prefix
// column and on draft column P_b + j exactly when j is i or an ancestor of i.
// mask_indptr[b] = T (kv_indptr[b] - kv_indptr[0]) + T^2 b, the closed form of
// the running sum of T N_b, so no scan is needed.
//
// Grid (gx, T, batch): workgroup (x, i, b) writes row i of request b, its
// threads striding over the 16-byte chunks the row overlaps. Interior chunks
// are one 16-byte store; the first and last chunk of a row, which it may
// share with its neighbours, are written byte by byte. HBM-bound (T N_b bytes
// written per request).

#include "tvmla_internal.h"

namespace tvmla {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void tree_mask_kernel(TreeMaskParams m) {
  const int b = blockIdx.z, i = blockIdx.y, T = m.num_draft;
  const int64_t base0 = m.kv_indptr[0];
  const int64_t P = m.kv_indptr[b + 1] - m.kv_indptr[b];
  const int64_t N = P + T;
  const int64_t ib = (int64_t)T * (m.kv_indptr[b] - base0) + (int64_t)T * T * b;  // mask_indptr[b]
  const int64_t o = ib + (int64_t)i * N;                                           // first byte of row i

  // bit j: draft node j is node i or an ancestor of it. The walk follows
  // parents only while they precede their child, so it ends in < T steps.
  __shared__ uint64_t anc_sh;
  if (threadIdx.x == 0) {
    uint64_t a = 0;
    int j = i;
    while (j >= 0) {
      a |= 1ull << j;
      const int pj = m.parents[(int64_t)b * T + j];
      j = pj < j ? pj : -1;
    }
    anc_sh = a;
  }
  __syncthreads();
  const uint64_t anc = anc_sh;
  auto byte_at = [&](int64_t p) -> uint8_t {  // p: column within the row
    return p < P ? 1 : (uint8_t)((anc >> (p - P)) & 1);
  };

  const int64_t k0 = o >> 4, k1 = (o + N - 1) >> 4;
  for (int64_t k = k0 + (int64_t)blockIdx.x * kThreads + threadIdx.x; k <= k1; k += (int64_t)gridDim.x * kThreads) {
    const int64_t c0 = k << 4;
    if (c0 >= o && c0 + 16 <= o + N) {
      uint4 v;
      if (c0 + 16 <= o + P) {
        v = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
      } else {
        uint32_t wds[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t wd = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) wd |= (uint32_t)byte_at(c0 + 4 * q + e - o) << (8 * e);
          wds[q] = wd;
        }
        v = make_uint4(wds[0], wds[1], wds[2], wds[3]);
      }
      *reinterpret_cast<uint4*>(m.mask + c0) = v;
    } else {
      for (int e = 0; e < 16; ++e) {
        const int64_t a = c0 + e;
        if (a >= o && a < o + N) m.mask[a] = byte_at(a - o);
      }
    }
  }
  if (blockIdx.x == 0 && i == 0 && threadIdx.x == 0) {
    m.mask_indptr[b] = (int32_t)ib;
    if (b == m.batch - 1) m.mask_indptr[m.batch] = (int32_t)(ib + (int64_t)T * N);
  }
}

}  // namespace

hipError_t launch_tree_mask(const TreeMaskParams& m, hipStream_t stream) {
  // about 2048 workgroups in all, at least one per row
  const int rows = m.batch * m.num_draft;
  const unsigned gx = (unsigned)std::max(1, std::min(128, (2048 + rows - 1) / rows));
  TreeMaskParams arg = m;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tree_mask_kernel),
                         dim3(gx, (unsigned)m.num_draft, (unsigned)m.batch), dim3(kThreads), args, 0, stream);
}

}  // namespace tvmla
