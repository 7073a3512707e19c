// KV defragmentation: copy each request's prefix rows into one contiguous
// run of cache slots and rewrite its kv_indices.
//
// page_size = 1 paging leaves a request's rows scattered over the pool, so
// every read of them is a gather of isolated 1152-byte rows ("The Plan
// Document: A Pivot Point in Custom CUDA Kernel Development", section
// "Context: The Bottleneck That Demanded a Custom Kernel"); compacting them
// is the plan's last phase (same page, section "Output Knowledge Created").
// Prefix position p of request b moves to slot dst_base[b] + p.
//
// Copy kernel: grid (gx, batch); workgroup x of request b copies rows
// j = x, x + gx, x + 2gx, ... of that request, flattened with their 16-byte
// chunks over the 256 threads (72 chunks per bf16 row, 144 per fp32 row), so
// each row is read and written as contiguous 16-byte pieces. Four pieces per
// thread are in flight at once. HBM-bound: per row 2 x 576 x elem_size bytes
// plus the 4-byte index.
//
// Index kernel: kv_indices_out[kv_indptr[b] + j] = dst_base[b] + j. It runs
// after the copy on the same stream, so kv_indices_out may alias kv_indices.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;

template <int kChunks>  // 16-byte chunks per row: 72 (bf16) or 144 (fp32)
__global__ __launch_bounds__(kThreads) void defrag_copy_kernel(DefragParams d) {
  const int b = blockIdx.y;
  const int gx = gridDim.x;
  const int i0 = d.kv_indptr[b];
  const int P = d.kv_indptr[b + 1] - i0;
  const int nrow = P > (int)blockIdx.x ? (P - (int)blockIdx.x + gx - 1) / gx : 0;  // rows of this workgroup
  const int64_t items = (int64_t)nrow * kChunks;
  const int64_t dbase = d.dst_base[b];
  const char* src = static_cast<const char*>(d.src);
  char* dst = static_cast<char*>(d.dst);
  for (int64_t w0 = threadIdx.x; w0 < items; w0 += (int64_t)kThreads * kInFlight) {
    uint4 v[kInFlight];
    int64_t doff[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t w = w0 + (int64_t)u * kThreads;
      doff[u] = -1;
      if (w < items) {
        const int i = (int)(w / kChunks);
        const int c = (int)(w - (int64_t)i * kChunks);
        const int j = (int)blockIdx.x + i * gx;
        const int64_t slot = d.kv_indices[i0 + j];
        v[u] = *reinterpret_cast<const uint4*>(src + slot * d.src_row_bytes + 16 * c);
        doff[u] = (dbase + j) * d.dst_row_bytes + 16 * c;
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (doff[u] >= 0) *reinterpret_cast<uint4*>(dst + doff[u]) = v[u];
  }
}

__global__ __launch_bounds__(kThreads) void defrag_index_kernel(DefragParams d) {
  const int b = blockIdx.y;
  const int i0 = d.kv_indptr[b];
  const int P = d.kv_indptr[b + 1] - i0;
  const int dbase = d.dst_base[b];
  for (int j = blockIdx.x * kThreads + threadIdx.x; j < P; j += gridDim.x * kThreads) d.indices_out[i0 + j] = dbase + j;
}

}  // namespace

hipError_t launch_defrag(const DefragParams& d, int elem_size, hipStream_t stream) {
  // about 2048 copy workgroups in all, at least one per request
  const unsigned gx = (unsigned)std::max(1, std::min(2048, (2048 + d.batch - 1) / d.batch));
  DefragParams arg = d;
  void* args[] = {&arg};
  const void* fn = elem_size == 2 ? reinterpret_cast<const void*>(&defrag_copy_kernel<kDKey * 2 / 16>)
                                  : reinterpret_cast<const void*>(&defrag_copy_kernel<kDKey * 4 / 16>);
  hipError_t e = hipLaunchKernel(fn, dim3(gx, (unsigned)d.batch), dim3(kThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned ix = (unsigned)std::max(1, std::min(256, (256 + d.batch - 1) / d.batch));
  return hipLaunchKernel(reinterpret_cast<const void*>(&defrag_index_kernel), dim3(ix, (unsigned)d.batch),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace tvmla
