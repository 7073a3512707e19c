// Internal declarations shared by the tvmla kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tvmla {

constexpr int kDLatent = 512;
constexpr int kDRope = 64;
constexpr int kDKey = kDLatent + kDRope;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything a split kernel needs; passed by value as one kernel argument.
struct SplitParams {
  const void* q_nope;
  int64_t qn_stride_tok, qn_stride_head;  // elements
  const void* q_rope;
  int64_t qr_stride_tok, qr_stride_head;  // elements
  const void* kv;
  int64_t kv_stride;  // elements per cache row
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* out_cache_loc;
  const uint8_t* mask;
  const int32_t* mask_indptr;
  int32_t batch, num_draft, num_heads, nsplit, min_chunk;
  int32_t chunk_align;  // chunks rounded up to a multiple of this (1: the pages' rule exactly)
  float sm_scale;
  float* o_part;    // [batch][nsplit][num_draft * num_heads][512]
  float* lse_part;  // [batch][nsplit][num_draft * num_heads]
  const int64_t* qo_indptr;  // null: num_draft tokens per request; else per-request token ranges
  float fold_log2;           // row-owner kernel: reference-max growth (log2 units) that triggers a fold
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  const int32_t* kv_indptr;  // may be null: read every split
  int32_t batch, num_draft, num_heads, nsplit, min_chunk;
  int32_t chunk_align;  // as SplitParams::chunk_align
  const int64_t* qo_indptr;  // null: num_draft tokens per request; else per-request token ranges
  void* out;
  float* lse;
};

struct DefragParams {
  const void* src;
  void* dst;
  int64_t src_row_bytes, dst_row_bytes;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* dst_base;
  int32_t* indices_out;
  int32_t batch;
};

struct TreeMaskParams {
  const int32_t* parents;    // [batch * num_draft], parent of node i within its request, -1 for the root
  const int32_t* kv_indptr;  // [batch + 1]
  uint8_t* mask;
  int32_t* mask_indptr;      // [batch + 1]
  int32_t batch, num_draft;
};

// Workspace regions (byte offsets from the workspace base).
struct WorkspaceLayout {
  size_t o_off, lse_off, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WorkspaceLayout workspace_layout(int64_t batch, int64_t num_draft, int64_t num_heads, int64_t nsplit) {
  const size_t rows = (size_t)batch * (size_t)nsplit * (size_t)num_draft * (size_t)num_heads;
  WorkspaceLayout w;
  w.o_off = 0;
  w.lse_off = align_up(rows * kDLatent * sizeof(float), 256);
  w.total = align_up(w.lse_off + rows * sizeof(float), 256);
  return w;
}

// Keys per split of a request with n keys: max(ceil(n / nsplit),
// min_chunk) rounded up to a multiple of align (align 1 and min_chunk 0
// give the pages' ceil(n / nsplit)).
__host__ __device__ inline int64_t split_chunk(int n, int nsplit, int min_chunk, int align) {
  int64_t chunk = ((int64_t)n + nsplit - 1) / nsplit;
  if (chunk < min_chunk) chunk = min_chunk;
  return (chunk + align - 1) / align * align;
}

// Key range [start, end) of split s of a request with n keys: split s
// starts at s * split_chunk(...).
__host__ __device__ inline void split_bounds(int n, int nsplit, int min_chunk, int align, int s, int& start,
                                             int& end) {
  const int64_t chunk = split_chunk(n, nsplit, min_chunk, align);
  const int64_t st = (int64_t)s * chunk;
  start = st < n ? (int)st : n;
  const int64_t en = st + chunk;
  end = en < n ? (int)en : n;
}

// Number of leading splits that hold keys under split_bounds.
__host__ __device__ inline int active_splits(int n, int nsplit, int min_chunk, int align) {
  if (n <= 0) return 0;
  const int64_t chunk = split_chunk(n, nsplit, min_chunk, align);
  const int64_t a = ((int64_t)n + chunk - 1) / chunk;
  return a < nsplit ? (int)a : nsplit;
}

// Draft tokens of request b and the index of its first one: num_draft and
// b * num_draft, or with qo_indptr its range qo_indptr[b] .. qo_indptr[b+1]
// (the count clamped to [0, num_draft]).
__device__ inline void request_tokens(const int64_t* qo_indptr, int num_draft, int b, int& Tb, int64_t& t0) {
  if (qo_indptr == nullptr) {
    Tb = num_draft;
    t0 = (int64_t)b * num_draft;
    return;
  }
  t0 = qo_indptr[b];
  const int64_t n = qo_indptr[b + 1] - t0;
  Tb = n < 0 ? 0 : (n > num_draft ? num_draft : (int)n);
}

// Request served by the (request, split) pairs of rank `rank`, longest
// request first. Workgroups start roughly in id order and pair indices grow
// with the id, so handing the first pairs to the requests with the most keys
// (all splits of a request are equally long) lets the short requests fill
// the compute units at the end: longest-processing-time-first list
// scheduling, where index order can leave a few long workgroups running
// alone. The order is a function of the device-side lengths, so the grid
// stays fixed. Rank of request j = number of requests with more keys, or as
// many keys and a lower index (a strict total order, so the ranks are a
// permutation and exactly one lane matches). Every lane of the wavefront
// must be active. Batches of one or of more than 64 keep index order.
__device__ inline int request_of_rank(const SplitParams& p, int rank) {
  if (p.batch <= 1 || p.batch > 64) return rank;
  const int lane = threadIdx.x & 63;
  int n = -1;
  if (lane < p.batch) {
    int Tb;
    int64_t t0;
    request_tokens(p.qo_indptr, p.num_draft, lane, Tb, t0);
    n = p.kv_indptr[lane + 1] - p.kv_indptr[lane] + Tb;
  }
  int above = 0;
  for (int j = 0; j < p.batch; ++j) {
    const int nj = __builtin_amdgcn_readlane(n, j);
    above += (nj > n || (nj == n && j < lane)) ? 1 : 0;
  }
  return __builtin_ctzll(__ballot(lane < p.batch && above == rank));
}

// fp32 -> bf16 with round to nearest even (a NaN stays a NaN): the
// hardware conversion, v_cvt_pk_bf16_f32, two values per instruction.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Four fp32 values as bf16 (round to nearest even), packed into 8 bytes.
__device__ inline uint2 pack_bf16x4(float a, float b, float c, float d) {
  uint2 u;
  u.x = pack_bf16x2(a, b);
  u.y = pack_bf16x2(c, d);
  return u;
}

// A split's partial output row in the workspace: a 2 KB slot (512 fp32). With
// bf16 queries the split kernels store the row as 512 bf16 in the slot's
// first 1 KB (half the bytes to write and to read back in the combine); with
// fp32 queries as 512 fp32.
__device__ inline uint16_t* partial_bf16(float* o_part, size_t prow) {
  return reinterpret_cast<uint16_t*>(o_part + prow * kDLatent);
}

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_split_scalar_bf16(const SplitParams& p, hipStream_t stream);
hipError_t launch_split_scalar_fp32(const SplitParams& p, hipStream_t stream);
hipError_t launch_split_mfma_bf16(const SplitParams& p, hipStream_t stream);
hipError_t launch_split_rows_bf16(const SplitParams& p, hipStream_t stream);
hipError_t launch_combine(const CombineParams& c, int dtype, hipStream_t stream);
hipError_t launch_defrag(const DefragParams& d, int elem_size, hipStream_t stream);
hipError_t launch_tree_mask(const TreeMaskParams& m, hipStream_t stream);

}  // namespace tvmla
