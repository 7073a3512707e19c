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
// Copy kernel: grid (gx, batch). A wavefront copies 8 consecutive prefix
// rows of request b at a time (units u = wavefront id, + stride, ...): lanes
// 0..7 load the 8 rows' slots, then the 8 x 72 16-byte chunks of the rows
// (8 x 144 for fp32) are spread over the 64 lanes, 9 (18) per lane, all
// loads issued before the first store. Each row is read and written as
// contiguous 16-byte pieces; the chunk values stay in registers. Loads and
// stores are non-temporal: the source rows are dead once copied and the
// destination is read only by later verify calls, so the copy should not
// displace what the L2s and the MALL hold (with ordinary loads, a copy that
// finds the MALL full of other dirty lines pays for their write-back).
// HBM-bound: per row 2 x 576 x elem_size bytes plus the 4-byte index.
//
// The index rewrite, kv_indices_out[kv_indptr[b] + j] = dst_base[b] + j, is
// done by the lane that reads kv_indices[kv_indptr[b] + j] for its unit,
// after that read: no other thread reads the element, so kv_indices_out may
// alias kv_indices, and no second launch is needed.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 8;  // rows per wavefront unit
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Nine chunks of a unit, chunk ids id = lane + 64 (K0 + k), k = 0..8: all
// nine loads first, then the stores (named registers, so nothing goes to
// scratch or LDS). Chunks past the unit's last row re-read that row and are
// not stored.
template <int kChunks, int K0>
__device__ __forceinline__ void copy_nine(const char* src, char* dst, const DefragParams& d, int64_t slot, int nr,
                                          int64_t drow0, int lane) {
#define TVMLA_CHUNK(k, r, c) \
  const int id##k = lane + 64 * (K0 + k), r = id##k / kChunks, c = id##k - r * kChunks
#define TVMLA_LOAD(k)                                                         \
  TVMLA_CHUNK(k, r##k, c##k);                                                 \
  const int64_t s##k = __shfl(slot, r##k < nr ? r##k : nr - 1, 64);          \
  const u32x4 v##k = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + s##k * d.src_row_bytes + 16 * c##k))
#define TVMLA_STORE(k) \
  if (r##k < nr) __builtin_nontemporal_store(v##k, reinterpret_cast<u32x4*>(dst + (drow0 + r##k) * d.dst_row_bytes + 16 * c##k))
  TVMLA_LOAD(0); TVMLA_LOAD(1); TVMLA_LOAD(2); TVMLA_LOAD(3); TVMLA_LOAD(4);
  TVMLA_LOAD(5); TVMLA_LOAD(6); TVMLA_LOAD(7); TVMLA_LOAD(8);
  TVMLA_STORE(0); TVMLA_STORE(1); TVMLA_STORE(2); TVMLA_STORE(3); TVMLA_STORE(4);
  TVMLA_STORE(5); TVMLA_STORE(6); TVMLA_STORE(7); TVMLA_STORE(8);
#undef TVMLA_STORE
#undef TVMLA_LOAD
#undef TVMLA_CHUNK
}

template <int kChunks>  // 16-byte chunks per row: 72 (bf16) or 144 (fp32)
__global__ __launch_bounds__(kThreads) void defrag_copy_kernel(DefragParams d) {
  static_assert(kRows * kChunks % (64 * 9) == 0, "a unit's chunks must come in nines per lane");
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i0 = d.kv_indptr[b];
  const int P = d.kv_indptr[b + 1] - i0;
  const int units = (P + kRows - 1) / kRows;
  const int64_t dbase = d.dst_base[b];
  const char* src = static_cast<const char*>(d.src);
  char* dst = static_cast<char*>(d.dst);
  for (int u = blockIdx.x * kWaves + wave; u < units; u += gridDim.x * kWaves) {
    const int j0 = u * kRows;
    const int nr = P - j0 < kRows ? P - j0 : kRows;  // rows of this unit (the request's last may be short)
    const int64_t slot = lane < nr ? (int64_t)d.kv_indices[i0 + j0 + lane] : 0;
    if (lane < nr) d.indices_out[i0 + j0 + lane] = (int32_t)(dbase + j0 + lane);  // after this lane's read
    copy_nine<kChunks, 0>(src, dst, d, slot, nr, dbase + j0, lane);
    if constexpr (kRows * kChunks == 2 * 64 * 9) copy_nine<kChunks, 9>(src, dst, d, slot, nr, dbase + j0, lane);
  }
}

}  // namespace

hipError_t launch_defrag(const DefragParams& d, int elem_size, hipStream_t stream) {
  // about 2048 copy workgroups (8,192 wavefronts) in all, at least one per request
  const unsigned gx = (unsigned)std::max(1, std::min(2048, (2048 + d.batch - 1) / d.batch));
  DefragParams arg = d;
  void* args[] = {&arg};
  const void* fn = elem_size == 2 ? reinterpret_cast<const void*>(&defrag_copy_kernel<kDKey * 2 / 16>)
                                  : reinterpret_cast<const void*>(&defrag_copy_kernel<kDKey * 4 / 16>);
  return hipLaunchKernel(fn, dim3(gx, (unsigned)d.batch), dim3(kThreads), args, 0, stream);
}

}  // namespace tvmla
