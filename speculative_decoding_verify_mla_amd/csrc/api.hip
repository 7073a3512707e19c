// C ABI of tvmla: host-side argument checks, workspace carving, launches.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and touches no device state. A call that passes enqueues exactly two
// kernels on the caller's stream (split, then combine); the launch
// configuration depends only on (batch, num_draft, num_heads, nsplit), so the
// pair can be captured into a hipGraph once and replayed while the metadata
// buffers change underneath ("The Architecture of Capture Safety", "The Core
// Problem": graph replay reissues the same launches at the same addresses).

#include "../../include/tvmla.h"
#include "tvmla_internal.h"

#include <algorithm>
#include <climits>
#include <mutex>

using namespace tvmla;

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Keys per tile of the MFMA split kernels: with TVMLA_FLAG_TILE_CHUNKS (or
// TVMLA_FLAG_TUNE_NSPLIT, which implies it) each split's chunk is rounded up
// to a multiple of it, so no split ends on a sliver of a tile.
constexpr int32_t kTileKeys = 64;
int32_t chunk_align(uint32_t flags) {
  return (flags & (TVMLA_FLAG_TUNE_NSPLIT | TVMLA_FLAG_TILE_CHUNKS)) ? kTileKeys : 1;
}

tvmla_status check_shape(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit) {
  if (batch < 1 || batch > 65535) return TVMLA_E_SHAPE;
  if (num_draft < 1 || num_draft > TVMLA_MAX_DRAFT) return TVMLA_E_SHAPE;
  if (num_heads < 1 || num_heads > TVMLA_MAX_HEADS) return TVMLA_E_SHAPE;
  if (nsplit < 1 || nsplit > TVMLA_MAX_NSPLIT) return TVMLA_E_SHAPE;
  return TVMLA_OK;
}

// Growth of a row's running max (log2 units) past which the row-owner
// kernel folds its accumulator into the workspace: 16 (probabilities stay
// below 2^16) unless the caller passes a finite threshold >= 0. Thresholds
// above 64 are taken as 64: a probability past 2^128 overflows fp32, and 64
// leaves the sums and the value products room. Results are the same for any
// threshold up to rounding; only the number of folds changes.
float fold_threshold(float fold_log2) {
  if (!(fold_log2 >= 0.f) || fold_log2 == INFINITY) return 16.f;
  return fold_log2 < 64.f ? fold_log2 : 64.f;
}

// Splits the split+combine entry points run with TVMLA_FLAG_TUNE_NSPLIT: the caller's nsplit doubled
// (up to TVMLA_MAX_NSPLIT) while the 128-row grid, batch * nsplit * ceil(T*H
// / 128) workgroups, would not cover the 256 compute units -- the shapes with
// few rows per request (8 heads per GPU) -- else halved as described below.
// A function of the sizes only, so
// the grid stays fixed for graph capture; results equal those at nsplit up
// to rounding (the LSE merge is exact in real arithmetic).
int32_t effective_nsplit(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit) {
  if (check_shape(batch, num_draft, num_heads, nsplit) != TVMLA_OK) return nsplit;
  const int64_t groups = ((int64_t)num_draft * num_heads + 127) / 128;
  int32_t ns = nsplit;
  auto grid = [&](int32_t n) { return (int64_t)batch * n * groups; };
  while (grid(ns) < 256 && 2 * ns <= TVMLA_MAX_NSPLIT) ns *= 2;
  if (ns != nsplit) return ns;
  // Fewer, longer splits where the grid has workgroups to spare. Each
  // workgroup pays a fixed cost (queries, split bounds and first tile
  // before the key loop, the partial-row writes after it) and every split
  // adds a partial row per query row for the combine to read. A grid of more
  // than one but at most two rounds of 256 workgroups runs as one round;
  // a larger one is halved while at least two rounds remain (batches of up
  // to 64 requests, which the split kernels serve longest request first) or
  // four (larger batches, served in index order), which still balances
  // ragged lengths over the compute units.
  if (grid(ns) > 256 && grid(ns) <= 512) {
    if (ns % 2 == 0 && grid(ns / 2) >= 256) ns /= 2;
  } else {
    const int64_t keep = batch <= 64 ? 512 : 1024;
    while (ns % 2 == 0 && grid(ns / 2) >= keep) ns /= 2;
  }
  return ns;
}

// bf16 kernel choice: the 128-row kernel does a third less work per row
// (staging, barriers and softmax exchange amortised over twice the rows),
// but launches half the workgroups of the 64-row one; it is taken when its
// grid still covers the 256 compute units.
int32_t auto_bf16(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit) {
  const int64_t rows = (int64_t)num_draft * num_heads;
  const int64_t wgs = (int64_t)batch * nsplit * ((rows + 127) / 128);
  return wgs >= 256 ? TVMLA_ALGO_ROWS : TVMLA_ALGO_MFMA;
}

// Library-owned scratch for tvmla_verify_noalloc: the split partials of
// callers that cannot allocate a workspace. Each device the library runs on
// holds its own copy until the process ends. In host code `noalloc_scratch`
// names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is ever handed to a kernel.
__device__ __align__(256) char noalloc_scratch[TVMLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// device's first call, then cached).
tvmla_status noalloc_scratch_address(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TVMLA_E_LAUNCH;
  // the kernels run on the stream's device; its scratch address is only
  // known here for the current device
  hipDevice_t sdev = dev;
  if (stream != nullptr && (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev)) return TVMLA_E_VALUE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || p == nullptr) return TVMLA_E_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TVMLA_OK;
}

}  // namespace

extern "C" {

size_t tvmla_workspace_bytes(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit) {
  if (check_shape(batch, num_draft, num_heads, nsplit) != TVMLA_OK) return 0;
  const int32_t ns = std::max(nsplit, effective_nsplit(batch, num_draft, num_heads, nsplit));
  return workspace_layout(batch, num_draft, num_heads, ns).total;
}

const char* tvmla_status_str(int32_t status) {
  switch (status) {
    case TVMLA_OK: return "ok";
    case TVMLA_E_NULLPTR: return "a required pointer is NULL";
    case TVMLA_E_SHAPE: return "a size or count is out of range";
    case TVMLA_E_DTYPE: return "unsupported dtype for this algorithm";
    case TVMLA_E_WORKSPACE: return "workspace missing or too small";
    case TVMLA_E_ALIGN: return "pointer or stride misaligned";
    case TVMLA_E_LAUNCH: return "kernel launch failed";
    case TVMLA_E_ALGO: return "unknown algorithm";
    case TVMLA_E_VALUE: return "a value argument is out of range (sm_scale, flags or fold threshold)";
    case TVMLA_E_INDEX: return "metadata holds an offset or slot out of range";
    default: return "unknown status";
  }
}

int32_t tvmla_version(void) { return 100; /* 0.1.0 */ }

int32_t tvmla_auto_algo(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit, int32_t dtype) {
  if (dtype != TVMLA_BF16 && dtype != TVMLA_FP32) return -TVMLA_E_DTYPE;
  const tvmla_status st = check_shape(batch, num_draft, num_heads, nsplit);
  if (st != TVMLA_OK) return -st;
  return dtype == TVMLA_BF16 ? auto_bf16(batch, num_draft, num_heads, nsplit) : TVMLA_ALGO_SCALAR;
}

int32_t tvmla_effective_nsplit(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit) {
  const tvmla_status st = check_shape(batch, num_draft, num_heads, nsplit);
  if (st != TVMLA_OK) return -st;
  return effective_nsplit(batch, num_draft, num_heads, nsplit);
}

// Host checks and parameter block shared by tvmla_verify_ex and
// tvmla_verify_partials. `out`/`lse` are only checked when need_out is set.
static tvmla_status prepare(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                            const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                            const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* out_cache_loc, const uint8_t* custom_mask,
                            const int32_t* mask_indptr, int32_t batch, int32_t num_draft, int32_t num_heads,
                            float sm_scale, int32_t nsplit, int32_t dtype, const void* out, const float* lse,
                            bool need_out, void* workspace, size_t workspace_bytes, int32_t& algo,
                            int32_t min_chunk, float fold_log2, SplitParams& p) {
  if (dtype != TVMLA_BF16 && dtype != TVMLA_FP32) return TVMLA_E_DTYPE;
  if (algo != TVMLA_ALGO_AUTO && algo != TVMLA_ALGO_SCALAR && algo != TVMLA_ALGO_MFMA && algo != TVMLA_ALGO_ROWS)
    return TVMLA_E_ALGO;
  if (algo == TVMLA_ALGO_AUTO) algo = dtype == TVMLA_BF16 ? auto_bf16(batch, num_draft, num_heads, nsplit) : TVMLA_ALGO_SCALAR;
  if ((algo == TVMLA_ALGO_MFMA || algo == TVMLA_ALGO_ROWS) && dtype != TVMLA_BF16) return TVMLA_E_DTYPE;
  if (!q_nope || !q_rope || !kv_cache || !kv_indptr || !kv_indices || !out_cache_loc || !custom_mask ||
      !mask_indptr)
    return TVMLA_E_NULLPTR;
  if (need_out && (!out || !lse)) return TVMLA_E_NULLPTR;
  if (!workspace) return TVMLA_E_WORKSPACE;
  tvmla_status st = check_shape(batch, num_draft, num_heads, nsplit);
  if (st != TVMLA_OK) return st;
  if (min_chunk < 0) return TVMLA_E_SHAPE;
  if (!(sm_scale > 0.f) || !(sm_scale < INFINITY)) return TVMLA_E_VALUE;
  if (fold_log2 != fold_log2) return TVMLA_E_VALUE;  // NaN
  if (kv_stride_row < TVMLA_D_KEY) return TVMLA_E_SHAPE;
  if (q_nope_stride_tok < 0 || q_nope_stride_head < 0 || q_rope_stride_tok < 0 || q_rope_stride_head < 0)
    return TVMLA_E_SHAPE;
  const int64_t esz = dtype == TVMLA_BF16 ? 2 : 4;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(workspace) ||
      (need_out && !aligned16(out)))
    return TVMLA_E_ALIGN;
  if ((kv_stride_row * esz) % 16 || (q_nope_stride_tok * esz) % 16 || (q_nope_stride_head * esz) % 16 ||
      (q_rope_stride_tok * esz) % 16 || (q_rope_stride_head * esz) % 16)
    return TVMLA_E_ALIGN;
  const WorkspaceLayout wl = workspace_layout(batch, num_draft, num_heads, nsplit);
  if (workspace_bytes < wl.total) return TVMLA_E_WORKSPACE;

  p.q_nope = q_nope;
  p.qn_stride_tok = q_nope_stride_tok;
  p.qn_stride_head = q_nope_stride_head;
  p.q_rope = q_rope;
  p.qr_stride_tok = q_rope_stride_tok;
  p.qr_stride_head = q_rope_stride_head;
  p.kv = kv_cache;
  p.kv_stride = kv_stride_row;
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.out_cache_loc = out_cache_loc;
  p.mask = custom_mask;
  p.mask_indptr = mask_indptr;
  p.batch = batch;
  p.num_draft = num_draft;
  p.num_heads = num_heads;
  p.nsplit = nsplit;
  p.min_chunk = min_chunk;
  p.chunk_align = 1;
  p.sm_scale = sm_scale;
  char* ws = static_cast<char*>(workspace);
  p.o_part = reinterpret_cast<float*>(ws + wl.o_off);
  p.lse_part = reinterpret_cast<float*>(ws + wl.lse_off);
  p.qo_indptr = nullptr;
  p.fold_log2 = fold_threshold(fold_log2);
  return TVMLA_OK;
}

static hipError_t launch_split(const SplitParams& p, int32_t algo, int32_t dtype, hipStream_t s) {
  if (algo == TVMLA_ALGO_MFMA) return launch_split_mfma_bf16(p, s);
  if (algo == TVMLA_ALGO_ROWS) return launch_split_rows_bf16(p, s);
  if (dtype == TVMLA_BF16) return launch_split_scalar_bf16(p, s);
  return launch_split_scalar_fp32(p, s);
}

// Split + combine; qo_indptr null = num_draft tokens per request. With
// TVMLA_FLAG_TUNE_NSPLIT the call runs effective_nsplit(...) splits, else
// exactly nsplit.
static tvmla_status verify_impl(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* out_cache_loc,
                                const uint8_t* custom_mask, const int32_t* mask_indptr, const int64_t* qo_indptr,
                                int32_t batch, int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                                int32_t dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream, int32_t algo, int32_t min_chunk, uint32_t flags, float fold_log2) {
  if (flags & ~(uint32_t)(TVMLA_FLAG_TUNE_NSPLIT | TVMLA_FLAG_TILE_CHUNKS)) return TVMLA_E_VALUE;
  SplitParams p;
  if (flags & TVMLA_FLAG_TUNE_NSPLIT) nsplit = effective_nsplit(batch, num_draft, num_heads, nsplit);
  tvmla_status st = prepare(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok,
                            q_rope_stride_head, kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc,
                            custom_mask, mask_indptr, batch, num_draft, num_heads, sm_scale, nsplit, dtype, out, lse,
                            true, workspace, workspace_bytes, algo, min_chunk, fold_log2, p);
  if (st != TVMLA_OK) return st;
  p.qo_indptr = qo_indptr;
  p.chunk_align = chunk_align(flags);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_split(p, algo, dtype, s) != hipSuccess) return TVMLA_E_LAUNCH;

  CombineParams c;
  c.o_part = p.o_part;
  c.lse_part = p.lse_part;
  c.kv_indptr = kv_indptr;
  c.batch = batch;
  c.num_draft = num_draft;
  c.num_heads = num_heads;
  c.nsplit = nsplit;
  c.min_chunk = min_chunk;
  c.chunk_align = p.chunk_align;
  c.qo_indptr = qo_indptr;
  c.out = out;
  c.lse = lse;
  if (launch_combine(c, dtype, s) != hipSuccess) return TVMLA_E_LAUNCH;
  return TVMLA_OK;
}

tvmla_status tvmla_verify_ex(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                             const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                             const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* out_cache_loc,
                             const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                             int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                             int32_t dtype, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream, int32_t algo, int32_t min_chunk,
                             uint32_t flags, float fold_log2) {
  return verify_impl(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok, q_rope_stride_head,
                     kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                     nullptr, batch, num_draft, num_heads, sm_scale, nsplit, dtype, out, lse, workspace,
                     workspace_bytes, stream, algo, min_chunk, flags, fold_log2);
}

tvmla_status tvmla_verify_ragged(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                 const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                 const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* out_cache_loc,
                                 const uint8_t* custom_mask, const int32_t* mask_indptr, const int64_t* qo_indptr,
                                 int32_t batch, int32_t max_draft, int32_t num_heads, float sm_scale,
                                 int32_t nsplit, int32_t dtype, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t algo, int32_t min_chunk,
                                 uint32_t flags, float fold_log2) {
  if (!qo_indptr) return TVMLA_E_NULLPTR;
  return verify_impl(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok, q_rope_stride_head,
                     kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                     qo_indptr, batch, max_draft, num_heads, sm_scale, nsplit, dtype, out, lse, workspace,
                     workspace_bytes, stream, algo, min_chunk, flags, fold_log2);
}

tvmla_status tvmla_verify_partials(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                   const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                   const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                   const int32_t* kv_indices, const int32_t* out_cache_loc,
                                   const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                                   int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                                   int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                                   int32_t algo, int32_t min_chunk, uint32_t flags, float fold_log2) {
  if (flags & ~(uint32_t)TVMLA_FLAG_TILE_CHUNKS) return TVMLA_E_VALUE;
  SplitParams p;
  tvmla_status st = prepare(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok,
                            q_rope_stride_head, kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc,
                            custom_mask, mask_indptr, batch, num_draft, num_heads, sm_scale, nsplit, dtype, nullptr,
                            nullptr, false, workspace, workspace_bytes, algo, min_chunk, fold_log2, p);
  if (st != TVMLA_OK) return st;
  p.chunk_align = chunk_align(flags);
  if (launch_split(p, algo, dtype, static_cast<hipStream_t>(stream)) != hipSuccess) return TVMLA_E_LAUNCH;
  return TVMLA_OK;
}

tvmla_status tvmla_verify(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                          const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                          const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* out_cache_loc,
                          const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                          int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                          int32_t dtype, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return verify_impl(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok, q_rope_stride_head,
                     kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                     nullptr, batch, num_draft, num_heads, sm_scale, nsplit, dtype, out, lse, workspace,
                     workspace_bytes, stream, TVMLA_ALGO_AUTO, 0, 0u, -1.f);
}

tvmla_status tvmla_verify_noalloc(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                  const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                  const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, const int32_t* out_cache_loc,
                                  const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                                  int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                                  int32_t dtype, void* out, float* lse, void* stream, int32_t algo,
                                  int32_t min_chunk, uint32_t flags, float fold_log2) {
  // every host check before the first HIP call, the scratch size included
  if (flags & ~(uint32_t)(TVMLA_FLAG_TUNE_NSPLIT | TVMLA_FLAG_TILE_CHUNKS)) return TVMLA_E_VALUE;
  if (check_shape(batch, num_draft, num_heads, nsplit) != TVMLA_OK) return TVMLA_E_SHAPE;
  const int32_t ns = (flags & TVMLA_FLAG_TUNE_NSPLIT) ? effective_nsplit(batch, num_draft, num_heads, nsplit) : nsplit;
  if (workspace_layout(batch, num_draft, num_heads, ns).total > (size_t)TVMLA_NOALLOC_SCRATCH_BYTES)
    return TVMLA_E_WORKSPACE;
  SplitParams probe;
  int32_t algo_checked = algo;
  tvmla_status st = prepare(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok,
                            q_rope_stride_head, kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc,
                            custom_mask, mask_indptr, batch, num_draft, num_heads, sm_scale, ns, dtype, out, lse, true,
                            reinterpret_cast<void*>(256), (size_t)TVMLA_NOALLOC_SCRATCH_BYTES, algo_checked,
                            min_chunk, fold_log2, probe);
  if (st != TVMLA_OK) return st;
  void* scratch = nullptr;
  st = noalloc_scratch_address(static_cast<hipStream_t>(stream), &scratch);
  if (st != TVMLA_OK) return st;
  return verify_impl(q_nope, q_nope_stride_tok, q_nope_stride_head, q_rope, q_rope_stride_tok, q_rope_stride_head,
                     kv_cache, kv_stride_row, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                     nullptr, batch, num_draft, num_heads, sm_scale, nsplit, dtype, out, lse, scratch,
                     (size_t)TVMLA_NOALLOC_SCRATCH_BYTES, stream, algo, min_chunk, flags, fold_log2);
}

tvmla_status tvmla_combine(const void* workspace, size_t workspace_bytes, const int32_t* kv_indptr,
                           int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit,
                           int32_t min_chunk, uint32_t flags, int32_t dtype, void* out, float* lse, void* stream) {
  if (flags & ~(uint32_t)TVMLA_FLAG_TILE_CHUNKS) return TVMLA_E_VALUE;
  if (dtype != TVMLA_BF16 && dtype != TVMLA_FP32) return TVMLA_E_DTYPE;
  if (!out || !lse) return TVMLA_E_NULLPTR;
  if (!workspace) return TVMLA_E_WORKSPACE;
  tvmla_status st = check_shape(batch, num_draft, num_heads, nsplit);
  if (st != TVMLA_OK) return st;
  if (min_chunk < 0) return TVMLA_E_SHAPE;
  if (!aligned16(workspace) || !aligned16(out)) return TVMLA_E_ALIGN;
  const WorkspaceLayout wl = workspace_layout(batch, num_draft, num_heads, nsplit);
  if (workspace_bytes < wl.total) return TVMLA_E_WORKSPACE;
  const char* ws = static_cast<const char*>(workspace);
  CombineParams c;
  c.o_part = reinterpret_cast<const float*>(ws + wl.o_off);
  c.lse_part = reinterpret_cast<const float*>(ws + wl.lse_off);
  c.kv_indptr = kv_indptr;
  c.batch = batch;
  c.num_draft = num_draft;
  c.num_heads = num_heads;
  c.nsplit = nsplit;
  c.min_chunk = min_chunk;
  c.chunk_align = chunk_align(flags);
  c.qo_indptr = nullptr;
  c.out = out;
  c.lse = lse;
  if (launch_combine(c, dtype, static_cast<hipStream_t>(stream)) != hipSuccess) return TVMLA_E_LAUNCH;
  return TVMLA_OK;
}

tvmla_status tvmla_check_metadata(const int32_t* kv_indptr, const int32_t* kv_indices, int64_t kv_indices_len,
                                  const int32_t* out_cache_loc, int64_t out_cache_loc_len, const int32_t* mask_indptr,
                                  int64_t mask_len, const int64_t* qo_indptr, int32_t batch, int32_t num_draft,
                                  int64_t num_slots, int32_t* bad_array, int64_t* bad_pos) {
  auto fail = [&](int32_t array, int64_t pos) {
    if (bad_array) *bad_array = array;
    if (bad_pos) *bad_pos = pos;
    return TVMLA_E_INDEX;
  };
  if (bad_array) *bad_array = TVMLA_META_NONE;
  if (bad_pos) *bad_pos = -1;
  if (!kv_indptr || !out_cache_loc || !mask_indptr || (!kv_indices && kv_indices_len > 0)) return TVMLA_E_NULLPTR;
  if (batch < 1 || batch > 65535 || num_draft < 1 || num_draft > TVMLA_MAX_DRAFT) return TVMLA_E_SHAPE;
  if (num_slots < 1 || kv_indices_len < 0 || out_cache_loc_len < 0 || mask_len < 0) return TVMLA_E_SHAPE;
  // offsets: kv_indptr non-decreasing inside kv_indices, prefixes short
  // enough that N_b = P_b + T_b fits the kernels' 32-bit key positions
  if (kv_indptr[0] < 0) return fail(TVMLA_META_KV_INDPTR, 0);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t P = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    if (P < 0 || P > INT32_MAX - TVMLA_MAX_DRAFT) return fail(TVMLA_META_KV_INDPTR, b + 1);
  }
  if (kv_indptr[batch] > kv_indices_len) return fail(TVMLA_META_KV_INDPTR, batch);
  if (qo_indptr) {
    if (qo_indptr[0] < 0) return fail(TVMLA_META_QO_INDPTR, 0);
    for (int32_t b = 0; b < batch; ++b)
      if (qo_indptr[b + 1] < qo_indptr[b]) return fail(TVMLA_META_QO_INDPTR, b + 1);
  }
  // slots
  for (int64_t j = kv_indptr[0]; j < kv_indptr[batch]; ++j)
    if (kv_indices[j] < 0 || kv_indices[j] >= num_slots) return fail(TVMLA_META_KV_INDICES, j);
  for (int32_t b = 0; b < batch; ++b) {
    int64_t t0 = (int64_t)b * num_draft, Tb = num_draft;
    if (qo_indptr) {  // the kernels clamp a request's token count to num_draft
      t0 = qo_indptr[b];
      Tb = std::min<int64_t>(qo_indptr[b + 1] - t0, num_draft);
    }
    for (int64_t t = t0; t < t0 + Tb; ++t) {
      if (t >= out_cache_loc_len) return fail(TVMLA_META_OUT_CACHE_LOC, t);
      if (out_cache_loc[t] < 0 || out_cache_loc[t] >= num_slots) return fail(TVMLA_META_OUT_CACHE_LOC, t);
    }
    // the request's [T_b][N_b] mask block must lie inside custom_mask
    const int64_t N = (int64_t)kv_indptr[b + 1] - kv_indptr[b] + Tb;
    if (mask_indptr[b] < 0 || mask_indptr[b] + Tb * N > mask_len) return fail(TVMLA_META_MASK_INDPTR, b);
  }
  return TVMLA_OK;
}

tvmla_status tvmla_defrag(const void* kv_src, int64_t src_stride_row, void* kv_dst, int64_t dst_stride_row,
                          const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* dst_base,
                          int32_t* kv_indices_out, int32_t batch, int32_t dtype, void* stream) {
  if (dtype != TVMLA_BF16 && dtype != TVMLA_FP32) return TVMLA_E_DTYPE;
  if (!kv_src || !kv_dst || !kv_indptr || !kv_indices || !dst_base || !kv_indices_out) return TVMLA_E_NULLPTR;
  if (batch < 1 || batch > 65535) return TVMLA_E_SHAPE;
  if (src_stride_row < TVMLA_D_KEY || dst_stride_row < TVMLA_D_KEY) return TVMLA_E_SHAPE;
  const int64_t esz = dtype == TVMLA_BF16 ? 2 : 4;
  if (!aligned16(kv_src) || !aligned16(kv_dst) || (src_stride_row * esz) % 16 || (dst_stride_row * esz) % 16)
    return TVMLA_E_ALIGN;
  DefragParams d;
  d.src = kv_src;
  d.dst = kv_dst;
  d.src_row_bytes = src_stride_row * esz;
  d.dst_row_bytes = dst_stride_row * esz;
  d.kv_indptr = kv_indptr;
  d.kv_indices = kv_indices;
  d.dst_base = dst_base;
  d.indices_out = kv_indices_out;
  d.batch = batch;
  if (launch_defrag(d, (int)esz, static_cast<hipStream_t>(stream)) != hipSuccess) return TVMLA_E_LAUNCH;
  return TVMLA_OK;
}

tvmla_status tvmla_tree_mask(const int32_t* parents, const int32_t* kv_indptr, int32_t batch, int32_t num_draft,
                             uint8_t* custom_mask, int32_t* mask_indptr, void* stream) {
  if (!parents || !kv_indptr || !custom_mask || !mask_indptr) return TVMLA_E_NULLPTR;
  if (batch < 1 || batch > 65535) return TVMLA_E_SHAPE;
  if (num_draft < 1 || num_draft > TVMLA_MAX_DRAFT) return TVMLA_E_SHAPE;
  TreeMaskParams m;
  m.parents = parents;
  m.kv_indptr = kv_indptr;
  m.mask = custom_mask;
  m.mask_indptr = mask_indptr;
  m.batch = batch;
  m.num_draft = num_draft;
  if (launch_tree_mask(m, static_cast<hipStream_t>(stream)) != hipSuccess) return TVMLA_E_LAUNCH;
  return TVMLA_OK;
}

}  // extern "C"
