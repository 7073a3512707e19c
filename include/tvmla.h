/*
 * tvmla.h -- tree-verify attention over an MLA latent KV cache, for AMD
 * Instinct MI355X (gfx950).
 *
 * One call computes the verify attention of a speculative-decoding draft tree:
 * every draft token of every request attends, with every head, to the request's
 * prefix keys and to the draft keys its visibility mask allows. This is the
 * call described on "The Architecture of Capture Safety: Designing a CUDA
 * Graph-Compatible Verify Kernel for SGLang", section "The Design Emerges": a
 * split-K flash-decode over a fixed number of splits (first insight), prefix
 * keys through kv_indices/kv_indptr and draft keys through out_cache_loc with
 * no concatenated copy (second insight), the raw custom_mask/mask_indptr
 * indexed in the kernel (third insight), prefix lengths derived on the device
 * from kv_indptr (fourth insight), and a workspace the caller allocates once
 * (fifth insight). The cache layout is MLA's: one latent row per token, shared
 * by every head, serving as the value and as the first 512 entries of the key
 * ("The Plan Document", section "The Design Reasoning").
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers unless stated otherwise; the
 *     caller owns every buffer (workspace included). The library allocates
 *     nothing, keeps no global mutable state, and never synchronises; each
 *     call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream). It is safe to capture into a hipGraph: the launch
 *     configuration depends only on the scalar arguments, so prefix lengths,
 *     tree shapes and masks may change between replays at fixed addresses.
 *   - Argument checks run on the host before anything is enqueued. On error
 *     the call returns a status != TVMLA_OK and enqueues nothing. Index
 *     CONTENTS (slots, offsets, mask bytes) are trusted: a slot outside the
 *     cache or an offset outside its array is undefined behaviour. A caller
 *     that cannot vouch for them runs tvmla_check_metadata on host copies
 *     first.
 *   - Per request b: P_b = kv_indptr[b+1] - kv_indptr[b] prefix keys, then
 *     the T = num_draft draft keys, N_b = P_b + T keys in that order.
 *     Row (t, h) with t = b*T + i is draft token i of request b, head h.
 *   - Results are deterministic: identical inputs give bit-identical outputs
 *     (no atomics in any reduction).
 */
#ifndef TVMLA_H
#define TVMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TVMLA_D_LATENT 512 /* latent width: the value, key entries [0, 512) */
#define TVMLA_D_ROPE 64    /* rope width: key entries [512, 576)            */
#define TVMLA_D_KEY 576
#define TVMLA_MAX_DRAFT 64
#define TVMLA_MAX_HEADS 128
#define TVMLA_MAX_NSPLIT 256

typedef enum { TVMLA_BF16 = 0, TVMLA_FP32 = 1 } tvmla_dtype;

typedef enum {
  TVMLA_OK = 0,
  TVMLA_E_NULLPTR = 1,   /* a required pointer is NULL                          */
  TVMLA_E_SHAPE = 2,     /* a size or count is out of range                      */
  TVMLA_E_DTYPE = 3,     /* unknown dtype, or a dtype the chosen algorithm lacks */
  TVMLA_E_WORKSPACE = 4, /* workspace NULL or smaller than tvmla_workspace_bytes */
  TVMLA_E_ALIGN = 5,     /* a pointer or stride breaks the alignment rules       */
  TVMLA_E_LAUNCH = 6,    /* the HIP runtime rejected a kernel launch             */
  TVMLA_E_ALGO = 7,      /* unknown algorithm selector                           */
  TVMLA_E_VALUE = 8,     /* sm_scale not finite and positive, unknown flag bits,
                            or a NaN fold threshold                            */
  TVMLA_E_INDEX = 9      /* tvmla_check_metadata: an offset or slot out of range */
} tvmla_status;

typedef enum {
  TVMLA_ALGO_AUTO = 0,   /* bf16 -> ROWS when batch * nsplit * ceil(num_draft *
                            num_heads / 128) >= 256 (nsplit = the split count the
                            call runs), else MFMA; fp32 -> SCALAR             */
  TVMLA_ALGO_SCALAR = 1, /* one wavefront per (row, split); fp32 FMA; any dtype */
  TVMLA_ALGO_MFMA = 2,   /* bf16 MFMA kernel, 64 query rows per workgroup       */
  TVMLA_ALGO_ROWS = 3    /* bf16 MFMA kernel, 128 query rows per workgroup, each
                            wavefront owning 32 rows outright; bf16 only       */
} tvmla_algo;

/*
 * Flags of tvmla_verify_ex and tvmla_verify_ragged.
 *
 * TVMLA_FLAG_TUNE_NSPLIT: run tvmla_effective_nsplit(batch, num_draft,
 *   num_heads, nsplit) splits instead of exactly nsplit -- more splits when
 *   the grid would leave compute units idle, fewer when it would take more
 *   than one round of workgroups -- and round each split's chunk up to whole
 *   64-key tiles: chunk = 64 * ceil(max(ceil(N_b / ns), min_chunk) / 64),
 *   ns the effective count, so no split ends on a sliver of a tile (trailing
 *   splits may then hold no keys; they return at once and are never read).
 *   Still a fixed function of the sizes, so a captured graph keeps its grid;
 *   the merged result equals the one at nsplit up to rounding (the
 *   log-sum-exp merge is exact in real arithmetic). Without it the call runs
 *   exactly the caller's nsplit with the pages' chunk, the fixed split count
 *   of "The Architecture of Capture Safety", section "The NSPLIT
 *   Calculation".
 */
#define TVMLA_FLAG_TUNE_NSPLIT 1u
/*
 * TVMLA_FLAG_TILE_CHUNKS: round each split's chunk up to whole 64-key tiles
 *   (as TVMLA_FLAG_TUNE_NSPLIT does) while keeping nsplit as given. Accepted
 *   by every verify entry point, tvmla_verify_partials and tvmla_combine, so
 *   the two separate steps can reproduce a tuned call's schedule exactly:
 *   tvmla_verify_partials + tvmla_combine at tvmla_effective_nsplit(...)
 *   splits with this flag launch what tvmla_verify_ex with
 *   TVMLA_FLAG_TUNE_NSPLIT launches.
 */
#define TVMLA_FLAG_TILE_CHUNKS 2u

/*
 * fold_log2 (tvmla_verify_ex, _ragged, _partials): TVMLA_ALGO_ROWS keeps
 * each row's softmax against a reference max and moves the reference --
 * folding the row's accumulator into its workspace slot -- when a block of
 * keys would take a probability above 2^fold_log2 against it (the row's
 * scaled max, in log2 units, outgrew the reference by more than fold_log2).
 * A negative or infinite value selects the default, 16 (every probability
 * stays below 2^16), and values above 64 are taken as 64 (larger ones would
 * let probabilities overflow fp32); NaN is rejected with TVMLA_E_VALUE.
 * Results are the same for any threshold up to rounding: only the number of
 * folds changes (small thresholds make folds frequent, which tests use to
 * exercise that path). Other algorithms ignore it.
 */

/*
 * Bytes of workspace a verify call needs: the per-split partial results ("The
 * Architecture of Capture Safety", "Assumptions and Their Validity", assumption
 * 3: a fixed workspace sized from batch and constants only). It depends only on
 * its arguments, never on sequence lengths. Returns 0 for out-of-range
 * arguments.
 *
 * The size covers both nsplit splits (the count tvmla_verify runs, and
 * tvmla_verify_partials and tvmla_combine take as given) and
 * tvmla_effective_nsplit(batch, num_draft, num_heads, nsplit) splits (the
 * count run with TVMLA_FLAG_TUNE_NSPLIT), so one workspace serves both.
 *
 * Layout (each region 256-byte aligned), R = num_draft*num_heads, for the
 * nsplit a call uses:
 *   o_part   [batch][nsplit][R] slots of 2 KB: split s's output, normalised
 *                                     by its own softmax sum -- 512 bf16
 *                                     (rounded to nearest even) in the
 *                                     slot's first 1 KB for bf16 queries,
 *                                     512 fp32 for fp32 queries (the
 *                                     128-row kernel also uses the whole
 *                                     slot as fp32 scratch while it runs)
 *   lse_part [batch][nsplit][R]       split s's natural-log sum of exp
 *                                     (-inf when the split sees no key)
 * Row r = i*num_heads + h. Only splits that hold keys are written; the
 * rest of the workspace is left as it was.
 */
size_t tvmla_workspace_bytes(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit);

/*
 * Verify attention, then the log-sum-exp combine of its splits.
 *
 * q_nope   [batch*num_draft, num_heads, 512] dtype; element (t, h, d) at
 *          q_nope + t*q_nope_stride_tok + h*q_nope_stride_head + d
 * q_rope   [batch*num_draft, num_heads, 64] dtype, same form with its own
 *          strides (a packed [.., .., 576] query passes as two views).
 *          Strides are in elements; the last dimension is contiguous.
 * kv_cache [num_slots, kv_stride_row] dtype; row s holds slot s's key:
 *          entries [0, 512) the latent (also the value), [512, 576) rope.
 * kv_indptr     int32 [batch+1]   offsets into kv_indices (prefix only)
 * kv_indices    int32 [kv_indptr[batch]]  cache slots of prefix keys
 * out_cache_loc int32 [batch*num_draft]   cache slots of draft keys
 *               (their rows are already written)
 * custom_mask   uint8, per request a row-major [num_draft][N_b] block at
 *               offset mask_indptr[b]; nonzero = visible
 * mask_indptr   int32 [batch+1]
 * sm_scale      multiplies the full 576-wide dot product; must be finite
 *               and positive (a softmax temperature), else TVMLA_E_VALUE
 * nsplit        splits per request, used exactly as given: split s covers
 *               keys [s*chunk, min((s+1)*chunk, N_b)), chunk =
 *               ceil(N_b/nsplit) ("The Architecture of Capture Safety",
 *               "The NSPLIT Calculation"); empty splits return at once. (tvmla_verify_ex with
 *               TVMLA_FLAG_TUNE_NSPLIT adapts the count to the GPU.)
 * out      [batch*num_draft, num_heads, 512] dtype, contiguous; bf16 output
 *          is rounded to nearest even
 * lse      [batch*num_draft, num_heads] fp32, contiguous: natural log of the
 *          sum of exp(score) over the visible keys. A row that sees no key
 *          gets out = 0 and lse = -inf.
 * workspace, workspace_bytes: at least tvmla_workspace_bytes(...) bytes;
 *          contents on entry are ignored.
 *
 * Alignment: q, kv_cache, out and workspace 16-byte aligned; q strides and
 * kv_stride_row multiples of 16 bytes; kv_stride_row >= 576.
 * Limits: 1 <= batch; 1 <= num_draft <= 64; 1 <= num_heads <= 128;
 * 1 <= nsplit <= 256.
 */
tvmla_status tvmla_verify(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                          const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                          const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* out_cache_loc,
                          const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                          int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                          int32_t dtype, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * tvmla_verify with four extra knobs (tvmla_verify is this call with
 * TVMLA_ALGO_AUTO, 0, 0, -1):
 *   algo       a tvmla_algo value (TVMLA_ALGO_AUTO is tvmla_verify's choice)
 *   min_chunk  lower bound on the per-split chunk: chunk =
 *              max(ceil(N_b/nsplit), min_chunk). 0 or 1 keeps the rule
 *              above exactly. A larger value leaves short requests fewer,
 *              longer splits (the launch is unchanged; surplus splits return
 *              at once), which cuts partial-result traffic; the result
 *              differs only by rounding.
 *   flags      TVMLA_FLAG_TUNE_NSPLIT and/or TVMLA_FLAG_TILE_CHUNKS (other
 *              bits: TVMLA_E_VALUE)
 *   fold_log2  the fold threshold described above (negative: default)
 */
tvmla_status tvmla_verify_ex(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                             const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                             const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* out_cache_loc,
                             const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                             int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                             int32_t dtype, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream, int32_t algo, int32_t min_chunk,
                             uint32_t flags, float fold_log2);

/*
 * tvmla_verify_ex for draft trees of different sizes per request: request b
 * has T_b = qo_indptr[b+1] - qo_indptr[b] draft tokens, query rows
 * qo_indptr[b] .. qo_indptr[b+1]-1 (the int64 token offsets named on "The
 * Architecture of Capture Safety: ...", section "Input Knowledge Required";
 * the ragged layout is this library's reading). Everything else is as for
 * tvmla_verify_ex with num_draft replaced by max_draft = the largest T_b:
 *   - N_b = P_b + T_b keys: the prefix, then out_cache_loc[qo_indptr[b] ..
 *     qo_indptr[b+1]-1];
 *   - custom_mask: per request a row-major [T_b][N_b] block at
 *     mask_indptr[b];
 *   - q_nope/q_rope/out/lse: qo_indptr[batch] token rows in all;
 *   - workspace: tvmla_workspace_bytes(batch, max_draft, num_heads, nsplit);
 *   - the launch depends only on the scalars (max_draft fixes the grid;
 *     row groups past a request's T_b return at once), so token counts may
 *     change between graph replays.
 * qo_indptr (int64 [batch+1], device) must be non-decreasing; a T_b above
 * max_draft is clamped to max_draft (the request's last tokens are ignored).
 */
tvmla_status tvmla_verify_ragged(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                 const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                 const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* out_cache_loc,
                                 const uint8_t* custom_mask, const int32_t* mask_indptr, const int64_t* qo_indptr,
                                 int32_t batch, int32_t max_draft, int32_t num_heads, float sm_scale,
                                 int32_t nsplit, int32_t dtype, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t algo, int32_t min_chunk,
                                 uint32_t flags, float fold_log2);

/*
 * For callers that cannot allocate: code under hipGraph capture that must
 * not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation. The same call as tvmla_verify_ex, minus workspace and
 * workspace_bytes: the split partials go to a scratch array the library
 * owns in device memory, TVMLA_NOALLOC_SCRATCH_BYTES (256 MiB) per device,
 * held from the library's load until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   - Limit: calls whose workspace (tvmla_workspace_bytes' layout at the
 *     split count the call runs: nsplit, or tvmla_effective_nsplit(...) with
 *     TVMLA_FLAG_TUNE_NSPLIT) exceeds the scratch return TVMLA_E_WORKSPACE
 *     and enqueue nothing. E.g. 16 draft tokens x 64 heads fit up to 120
 *     splits of one request (the tuned 185k-context call runs 32).
 *   - All calls on one device share that device's array; it keeps the last
 *     call's partials, and nothing in it needs clearing between calls.
 *     Calls that overlap on one device (different streams, or host threads
 *     enqueueing concurrently) race on it: serialise them.
 *   - The first call on a device looks the array's device address up (with
 *     that device current) and caches it; `stream` must belong to the
 *     current device (else TVMLA_E_VALUE).
 * Other arguments, checks and results: as tvmla_verify_ex.
 */
#define TVMLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
tvmla_status tvmla_verify_noalloc(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                  const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                  const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, const int32_t* out_cache_loc,
                                  const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                                  int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                                  int32_t dtype, void* out, float* lse, void* stream, int32_t algo,
                                  int32_t min_chunk, uint32_t flags, float fold_log2);

/*
 * The split step alone: the same arguments as tvmla_verify_ex without out
 * and lse; nsplit is always used as given, so flags may only hold
 * TVMLA_FLAG_TILE_CHUNKS (else TVMLA_E_VALUE). It enqueues only the split
 * kernel, which leaves every non-empty split's partial result in the
 * workspace (layout under tvmla_workspace_bytes); tvmla_combine with the same
 * kv_indptr, nsplit, min_chunk and flags then produces exactly what
 * tvmla_verify_ex does at that split count. Callers that merge partials from
 * several sources, or that time the two steps apart, use the pair.
 */
tvmla_status tvmla_verify_partials(const void* q_nope, int64_t q_nope_stride_tok, int64_t q_nope_stride_head,
                                   const void* q_rope, int64_t q_rope_stride_tok, int64_t q_rope_stride_head,
                                   const void* kv_cache, int64_t kv_stride_row, const int32_t* kv_indptr,
                                   const int32_t* kv_indices, const int32_t* out_cache_loc,
                                   const uint8_t* custom_mask, const int32_t* mask_indptr, int32_t batch,
                                   int32_t num_draft, int32_t num_heads, float sm_scale, int32_t nsplit,
                                   int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                                   int32_t algo, int32_t min_chunk, uint32_t flags, float fold_log2);

/*
 * The combine step alone: merge per-split partials laid out as in
 * tvmla_workspace_bytes (the reduce of "The Architecture of Capture Safety",
 * "The Design Emerges", first insight). out = sum_s w_s o_s / sum_s w_s with
 * w_s = exp(lse_s - max lse), lse = max lse + log(sum_s w_s).
 *
 * If kv_indptr is non-NULL, split s of request b is read only when it holds
 * keys under the schedule above (N_b = kv_indptr[b+1]-kv_indptr[b]+num_draft,
 * chunk = max(ceil(N_b/nsplit), min_chunk), rounded up to whole 64-key tiles
 * with TVMLA_FLAG_TILE_CHUNKS, the only flag accepted); other splits are
 * never read.
 * If kv_indptr is NULL every split is read and a split with lse = -inf
 * weighs nothing. A row whose splits are all -inf gets out = 0, lse = -inf.
 * workspace: as for tvmla_verify (read only here).
 */
tvmla_status tvmla_combine(const void* workspace, size_t workspace_bytes, const int32_t* kv_indptr,
                           int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit,
                           int32_t min_chunk, uint32_t flags, int32_t dtype, void* out, float* lse, void* stream);

/*
 * KV defragmentation: copy every request's prefix rows into one contiguous
 * run of cache slots and rewrite its indices. page_size = 1 paging scatters
 * a request's rows over the pool, so every read of them gathers isolated
 * rows ("The Plan Document: A Pivot Point in Custom CUDA Kernel
 * Development", section "Context: The Bottleneck That Demanded a Custom
 * Kernel"); compaction is the plan's last phase (same page, section "Output
 * Knowledge Created"). The interface is this library's own reading:
 *
 *   for b < batch, p < P_b = kv_indptr[b+1] - kv_indptr[b]:
 *     kv_dst[dst_base[b] + p][0:576] = kv_src[kv_indices[kv_indptr[b] + p]][0:576]
 *     kv_indices_out[kv_indptr[b] + p] = dst_base[b] + p
 *
 * kv_src, kv_dst   caches of `dtype` (rows of src_stride_row / dst_stride_row
 *                  elements, >= 576; entries past 576 are not touched). They
 *                  may be the same cache.
 * kv_indptr, kv_indices   as for tvmla_verify (read only).
 * dst_base         int32 [batch]: first destination slot of each request.
 * kv_indices_out   int32 [kv_indptr[batch]]: the rewritten indices; may be
 *                  kv_indices itself (each index is rewritten after it has
 *                  been read, by the thread that read it).
 * Draft rows (out_cache_loc) are not moved. The destination runs must not
 * overlap each other or any source row of the same call (the caller picks
 * free slots); overlapping runs are undefined behaviour.
 * Alignment: caches 16-byte aligned, row strides multiples of 16 bytes.
 * Limits: 1 <= batch <= 65535. Enqueues one kernel on `stream`.
 */
tvmla_status tvmla_defrag(const void* kv_src, int64_t src_stride_row, void* kv_dst, int64_t dst_stride_row,
                          const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* dst_base,
                          int32_t* kv_indices_out, int32_t batch, int32_t dtype, void* stream);

/*
 * Visibility mask of the draft trees, built on the device (no host
 * marshaling; capture-safe). A DDTree drafter proposes a tree of draft tokens
 * verified in one pass, which needs a mask of which draft token sees which
 * key ("The Architecture of Capture Safety: Designing a CUDA
 * Graph-Compatible Verify Kernel for SGLang", section "Input Knowledge
 * Required", DDTree paragraph); this writes it in the raw custom_mask +
 * mask_indptr form tvmla_verify reads (same page, section "The Design
 * Emerges", third insight).
 *
 * parents      int32 [batch * num_draft]: parents[b*T + i] is the parent of
 *              draft node i of request b (-1 for the root, node 0); a parent
 *              precedes its child (parents[b*T + i] < i). A parent that does
 *              not precede its child ends the walk there (no hang).
 * kv_indptr    int32 [batch+1], as for tvmla_verify (P_b prefix keys).
 * custom_mask  uint8 output, sum_b T * (P_b + T) bytes: row i of request b
 *              is 1 on every prefix column and on draft column P_b + j iff j
 *              is i or an ancestor of i, 0 elsewhere.
 * mask_indptr  int32 [batch+1] output: mask_indptr[b] = T*(kv_indptr[b] -
 *              kv_indptr[0]) + T*T*b; the total must stay below 2^31.
 * Limits: 1 <= batch <= 65535; 1 <= num_draft <= 64. One kernel on `stream`.
 */
tvmla_status tvmla_tree_mask(const int32_t* parents, const int32_t* kv_indptr, int32_t batch, int32_t num_draft,
                             uint8_t* custom_mask, int32_t* mask_indptr, void* stream);

/* Which array tvmla_check_metadata found at fault. */
typedef enum {
  TVMLA_META_NONE = 0,
  TVMLA_META_KV_INDPTR = 1,
  TVMLA_META_KV_INDICES = 2,
  TVMLA_META_OUT_CACHE_LOC = 3,
  TVMLA_META_MASK_INDPTR = 4,
  TVMLA_META_QO_INDPTR = 5
} tvmla_meta_array;

/*
 * Host-side check of the metadata a verify call reads raw (SGLang's
 * metadata buffers, which the kernel consumes as they are: "The
 * Architecture of Capture Safety: ...", section "The Core Problem"). All
 * pointers here are HOST pointers (copies of what the device call will
 * get); nothing is enqueued and no HIP call is made. Returns TVMLA_OK when
 * every offset and slot a call with these arguments (tvmla_verify/_ex when
 * qo_indptr is NULL, tvmla_verify_ragged with max_draft = num_draft
 * otherwise) would read lies inside its array, else TVMLA_E_INDEX and, when
 * the pointers are non-NULL, the faulty array (tvmla_meta_array) in
 * *bad_array and the element position in *bad_pos (-1 if none). Checks, in
 * this order:
 *   kv_indptr   kv_indptr[0] >= 0; 0 <= P_b <= INT32_MAX - 64 (so N_b fits
 *               32 bits); kv_indptr[batch] <= kv_indices_len
 *   qo_indptr   (if given) qo_indptr[0] >= 0 and non-decreasing (a T_b above
 *               num_draft is clamped, as the verify calls do)
 *   kv_indices  every entry in [kv_indptr[0], kv_indptr[batch]) is a slot
 *               in [0, num_slots)
 *   per request b, in order: out_cache_loc positions of its T_b draft tokens
 *               inside out_cache_loc_len and their slots in [0, num_slots);
 *               then mask_indptr[b] >= 0 and mask_indptr[b] + T_b * N_b <=
 *               mask_len
 * Other errors: TVMLA_E_NULLPTR (kv_indptr, out_cache_loc, mask_indptr
 * NULL, or kv_indices NULL with kv_indices_len > 0), TVMLA_E_SHAPE (batch
 * outside [1, 65535], num_draft outside [1, 64], num_slots < 1, a negative
 * length).
 */
tvmla_status tvmla_check_metadata(const int32_t* kv_indptr, const int32_t* kv_indices, int64_t kv_indices_len,
                                  const int32_t* out_cache_loc, int64_t out_cache_loc_len, const int32_t* mask_indptr,
                                  int64_t mask_len, const int64_t* qo_indptr, int32_t batch, int32_t num_draft,
                                  int64_t num_slots, int32_t* bad_array, int64_t* bad_pos);

/* A static, human-readable name for a status code (host pointer, never NULL). */
const char* tvmla_status_str(int32_t status);

/* Library version: major*10000 + minor*100 + patch. */
int32_t tvmla_version(void);

/*
 * The algorithm TVMLA_ALGO_AUTO resolves to for these sizes and dtype (a
 * tvmla_algo value), nsplit being the split count the call runs (with
 * TVMLA_FLAG_TUNE_NSPLIT, tvmla_effective_nsplit(...)), or a negative
 * tvmla_status for out-of-range sizes or an unknown dtype. Host only; no
 * HIP call.
 */
int32_t tvmla_auto_algo(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit, int32_t dtype);

/*
 * The split count tvmla_verify_ex and tvmla_verify_ragged run with
 * TVMLA_FLAG_TUNE_NSPLIT for these sizes. With G = batch * nsplit *
 * ceil(num_draft * num_heads / 128) workgroups of the 128-row kernel:
 * nsplit doubled (up to TVMLA_MAX_NSPLIT) while G < 256, i.e. while the
 * requested grid would leave compute units idle (few rows per request, e.g.
 * 8 heads per GPU); else, for 256 < G <= 512, nsplit / 2 when nsplit is
 * even and G / 2 >= 256 (one round of longer splits instead of two rounds,
 * each workgroup paying its fixed cost before and after the key loop once);
 * else nsplit halved while it is even and the halved grid still has >= 512
 * workgroups when batch <= 64 (at least two rounds: such batches are served
 * longest request first) or >= 1024 for larger batches (four rounds); fewer
 * partial rows to write and combine. A fixed function of the sizes, so a
 * captured graph keeps its grid; the workspace size from
 * tvmla_workspace_bytes accounts for it. tvmla_verify, tvmla_verify_partials
 * and tvmla_combine use nsplit exactly as given.
 * Negative tvmla_status for out-of-range sizes. Host only.
 */
int32_t tvmla_effective_nsplit(int32_t batch, int32_t num_draft, int32_t num_heads, int32_t nsplit);

#ifdef __cplusplus
}
#endif

#endif /* TVMLA_H */
