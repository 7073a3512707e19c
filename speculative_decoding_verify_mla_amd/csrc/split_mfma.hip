// bf16 MFMA split kernel for gfx950.
//
// Work unit: one workgroup = (request b, split s, group of 64 query rows). A
// request's rows are r = i*H + h (draft token i, head h). Every row of a
// request attends to the same keys, so one key tile staged in LDS feeds all 64
// rows of the group -- the "read the shared latent once, use it for many heads"
// reuse of "The Plan Document", section "The Design Reasoning" (variants 2 and
// 3), taken further because the products run on the matrix cores.
//
// Tile = 64 keys, staged whole with direct global->LDS loads (16 bytes per
// lane, no registers involved), double-buffered: while the four wavefronts
// work on tile t, tile t+1 is already in flight. In LDS a tile is a latent
// region (64 keys x 1024 bytes; one wavefront-wide load per key) followed by
// a rope region (64 keys x 128 bytes; one load per 8 keys). Within a key's
// row the 16-byte pieces are XOR-swizzled by a function of the key, so the
// MFMA operand reads of consecutive keys hit different LDS banks.
//
// Wavefront w = (row block rb = w & 1, key half kh = w >> 1):
//   scores   S^T = K Q^T for its 32 keys x 32 rows with
//            v_mfma_f32_32x32x16_bf16 (A = key rows from LDS, B = the row
//            block's queries, held in registers for the whole split);
//   softmax  per-row max over the 64-key tile via a 512-byte LDS exchange,
//            probabilities rounded to bf16 and shared through LDS in the
//            layout the next MFMA consumes as its B operand;
//   values   O^T += V^T P^T for latent entries [128w, 128w+128) of BOTH row
//            blocks, so each V^T operand read from LDS serves 64 rows. V^T is
//            read straight from the row-major key tile with the gfx950
//            transpose read (ds_read_b64_tr_b16: within each 16-lane group,
//            four 64-bit pieces of four rows come back as their columns).
//   The output block O^T (128 latent entries x 64 rows, fp32) stays in
//   registers across the split.
//
// Schedule and indexing follow "The Architecture of Capture Safety", "The
// Design Emerges": split s of a request with N keys covers [s*chunk,
// min((s+1)*chunk, N)), chunk = ceil(N / nsplit), an empty split returns at
// once (first insight); a key's slot comes from kv_indices (prefix) or
// out_cache_loc (draft) (second); the mask byte is custom_mask[mask_indptr[b] +
// i*N + p] (third); P_b comes from kv_indptr (fourth). The online softmax
// (running max, running sum, rescaled accumulator; "The Architecture of Capture
// Safety", "Input Knowledge Required") rescales the accumulator only when a
// row's running max grows by more than 2^8 since the last rescale, which keeps
// every probability below 256; the normalised result is the same.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
#define TVMLA_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

constexpr int kRowsWG = 64;   // query rows per workgroup (2 blocks of 32)
constexpr int kKT = 64;       // keys per tile (2 halves of 32)
constexpr int kLatRow = 1024; // bytes of one key's latent part in LDS (64 pieces of 16 B)
constexpr int kRopeRow = 128; // bytes of one key's rope part in LDS (8 pieces of 16 B)
constexpr int kTileLat = kKT * kLatRow;
constexpr int kTileBytes = kTileLat + kKT * kRopeRow;  // 73,728 bytes per tile buffer
constexpr int kQSteps = kDKey / 16;                    // 36 k-steps of 16 over the key width
constexpr float kRescaleLog2 = 8.f;                    // lazy-rescale threshold (log2 units)
constexpr int kRing = 6;                               // score operand reads in flight per wavefront

// Piece swizzle of key k (LDS serves 256 bytes = 16 pieces per cycle): the
// low two key bits go to piece bits 2..3 and key bits 2..3 to piece bits
// 0..1. Over 16 consecutive keys (the 16 lanes of one score-operand read
// cycle) it is a permutation of 0..15, and for the 4 consecutive keys x 4
// adjacent pieces a cycle of transposed reads covers it yields 16 distinct
// slots. Latent pieces XOR it (staying inside their aligned group of 16).
__host__ __device__ constexpr int piece_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
constexpr int kSwzHi = piece_swz(8) ^ piece_swz(0);  // swz(k + 8) ^ swz(k) for k % 16 < 8

// Workgroup barrier for LDS exchanges: waits only for this wavefront's LDS
// operations (lgkmcnt), not for its global loads -- the next tile's
// direct-to-LDS loads stay in flight across it. (__syncthreads() would add a
// workgroup fence, i.e. a wait for every outstanding global load.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier at the top of a tile: this wavefront's loads into the tile have
// landed (vmcnt) and so, after the barrier, have everyone else's.
// The wait is the compiler builtin (vmcnt(0) expcnt(7) lgkmcnt(0) in the
// gfx9 encoding) so the compiler knows every earlier load has completed.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_barrier" ::: "memory");
}

// Transposed LDS read (ds_read_b64_tr_b16) issued through inline asm. The
// compiler treats the builtin as touching any LDS location and would wait
// for every in-flight direct-to-LDS load before it; here the caller waits
// for the result explicitly (TVMLA_LDS_WAIT) before using it.
__device__ __forceinline__ i16x4_t tr_read(const char* lds_ptr) {
  const uint32_t a = (uint32_t)(uintptr_t)TVMLA_LDS(const char, lds_ptr);
  i16x4_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
  return r;
}

__device__ __forceinline__ u32x4_t lds_read128(const void* lds_ptr) {
  const uint32_t a = (uint32_t)(uintptr_t)TVMLA_LDS(const char, lds_ptr);
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
  return r;
}

// Wait for all outstanding LDS reads, with one value-product group's
// operand registers (lo[4], hi[4], pb[2]) tied to the wait so no use of them
// can be scheduled before it; TVMLA_PIN is the same ordering point without
// the wait. Nothing else touches those registers between the asm reads and
// the wait: they are the asm statements' own outputs and inputs.
#define TVMLA_TIE10(lo, hi, pb)                                                                                 \
  "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]), "+v"(hi[0]), "+v"(hi[1]), "+v"(hi[2]), "+v"(hi[3]),        \
      "+v"(pb[0]), "+v"(pb[1])
#define TVMLA_LDS_WAIT(lo, hi, pb) asm volatile("s_waitcnt lgkmcnt(0)" : TVMLA_TIE10(lo, hi, pb))
#define TVMLA_PIN(lo, hi, pb) asm volatile("" : TVMLA_TIE10(lo, hi, pb))
#define TVMLA_LDS_WAIT_F(lo, hi, pb, f) asm volatile("s_waitcnt lgkmcnt(0)" : TVMLA_TIE10(lo, hi, pb), "+v"(f))

// Score MFMA with the query operand read straight from AGPRs, where the
// queries live for the whole split (the builtin would copy each operand to
// VGPRs first). Back-to-back steps accumulate into the same registers, which
// needs no wait states; TVMLA_MFMA_DRAIN adds the wait states an XDL result
// needs before vector instructions may read it (the compiler cannot see
// through the asm, so they are spelled out: 24, twice what 8 passes need).
#define TVMLA_MFMA_QK_FIRST(acc, a, q) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(q))
#define TVMLA_MFMA_QK(acc, a, q) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(q))
#define TVMLA_MFMA_DRAIN(acc) asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc))

// Score operand read (ds_read_b128) whose completion the caller waits for
// with wait_lgkm_tied: "at most n LDS operations still outstanding", n being
// the number of this wavefront's LDS reads issued after it. LDS operations
// complete in order, so further LDS operations the compiler places in
// between only make the wait stricter.
__device__ __forceinline__ bf16x8_t frag_read(uint32_t lds_addr) {
  bf16x8_t r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_lgkm_n(bf16x8_t& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "n"(N));
}
__device__ __forceinline__ void wait_lgkm_tied(bf16x8_t& r, int n) {
  switch (n) {
    case 0: wait_lgkm_n<0>(r); break;
    case 1: wait_lgkm_n<1>(r); break;
    case 2: wait_lgkm_n<2>(r); break;
    case 3: wait_lgkm_n<3>(r); break;
    case 4: wait_lgkm_n<4>(r); break;
    case 5: wait_lgkm_n<5>(r); break;
    case 6: wait_lgkm_n<6>(r); break;
    default: wait_lgkm_n<7>(r); break;
  }
}

// An opaque copy of a value: the compiler cannot see through it, so
// addresses derived from it are computed where they are used instead of
// being hoisted out of the tile loop and kept in registers for its whole
// length.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ inline uint4 as_u4(bf16x8_t v) { return __builtin_bit_cast(uint4, v); }

__device__ inline bf16x8_t cat4(i16x4_t lo, i16x4_t hi) {
  typedef __attribute__((ext_vector_type(8))) short i16x8_t;
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Direct-to-LDS loads of one 64-key tile into `dst`, spread one load at a
// time over the previous tile's compute (a burst of loads would stall the
// issuing wavefront until the texture path drains it). slot_reg holds, in
// lane k, the cache slot of the tile's key k.
//   latent: key k = 16 wave + u (u = 0..15); the key's cache-row address,
//           which lane k holds in (ra_hi, ra_lo), goes to scalar registers
//           as the load's base and lane l loads piece l ^ swz(k) (a 32-bit
//           lane offset) into LDS piece l of the key's 1024-byte latent row;
//   rope:   keys 8v..8v+7 (v = 2 wave + u, u = 0..1), 128 contiguous bytes
//           each: lane l serves key k = 8v + l/8 and stores its 16-byte
//           piece (l%8) ^ (k%8) at position l%8 of the key's 128-byte rope
//           row, so a score read of one piece over 8 consecutive keys hits
//           8 different bank groups. `row` is lane l's source row, the
//           cache row of key k (fetched from lane k with a lane shuffle).
// Both load non-temporally (cache policy 2, `nt`): a cold call whose loads
// allocate in a MALL full of other dirty lines pays for their write-back (8
// heads: cold call 158 -> 134 us at 64 splits; warm 126 -> 130 us, the two
// row groups' shared key lines leaving the L2 sooner).
__device__ __forceinline__ void stage_key(char* dst, uint32_t ra_lo, uint32_t ra_hi, int wave, int lane, int u) {
  const int k = 16 * wave + u;  // swz(k) depends on u only
  const uint64_t row_addr = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(ra_hi, k) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(ra_lo, k);
  const char* src = reinterpret_cast<const char*>(row_addr) + ((lane ^ piece_swz(k)) << 4);
  __builtin_amdgcn_global_load_lds(src, TVMLA_LDS(void, dst + k * kLatRow), 16, 0, 2);
}

__device__ __forceinline__ void stage_rope(char* dst, const char* row, int wave, int lane, int u) {
  const int v = 2 * wave + u;
  const char* src = row + kDLatent * 2 + 16 * ((lane & 7) ^ (lane >> 3));
  __builtin_amdgcn_global_load_lds(src, TVMLA_LDS(void, dst + kTileLat + v * 8 * kRopeRow), 16, 0, 2);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_mfma_kernel(SplitParams p, int groups, int pairs) {
  __shared__ __attribute__((aligned(16))) char kb0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char kb1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint4 pex[4 * 2 * 64];  // P^T operands: [wave][k-step][lane]
  __shared__ float mex[4 * 32];                                   // per-wavefront row maxima / sums
  __shared__ __attribute__((aligned(16))) int rescale_flag[4];    // per wavefront: a row outgrew m_ref

  // Workgroup ids reach the 8 XCDs round-robin (id % 8). Every row group of
  // one (request, split) pair gets the same id % 8, so the pair's key rows
  // are fetched from HBM once and re-read from that XCD's L2.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int kq = id >> 3;
  const int jq = kq / groups;
  const int g = kq - jq * groups;
  const int pair = xcd + 8 * jq;
  if (pair >= pairs) return;
  const int b = request_of_rank(p, pair / p.nsplit);
  const int s = pair - (pair / p.nsplit) * p.nsplit;

  const int Rw = p.num_draft * p.num_heads;  // partial-row stride of the workspace
  int Tb;
  int64_t tb;  // draft tokens of request b, and the first one
  request_tokens(p.qo_indptr, p.num_draft, b, Tb, tb);
  const int R = Tb * p.num_heads;
  if (g * kRowsWG >= R) return;  // a shorter tree leaves this row group empty
  const int ip0 = p.kv_indptr[b];
  const int P = p.kv_indptr[b + 1] - ip0;
  const int N = P + Tb;
  int start, end;
  split_bounds(N, p.nsplit, p.min_chunk, p.chunk_align, s, start, end);
  if (start >= end) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5;   // which 8-wide half of each 16-wide k-step this lane feeds
  const int col = lane & 31;  // MFMA column = query row within the row block
  const int rb = wave & 1;    // row block whose scores this wavefront computes
  const int kh = wave >> 1;   // key half of each tile it scores

  // This lane's scoring row. A row past the end computes on row R-1's data
  // (each MFMA column is independent) and is never written.
  const int r = g * kRowsWG + rb * 32 + col;
  const int rr = r < R ? r : R - 1;
  const int i = rr / p.num_heads;
  const int h = rr - i * p.num_heads;
  const int64_t t = tb + i;

  // Q^T operands: query row `col` of block rb, key entries [16ks + 8hf, +8).
  bf16x8_t qf[kQSteps];
  {
    const uint16_t* qn = static_cast<const uint16_t*>(p.q_nope) + t * p.qn_stride_tok + h * p.qn_stride_head + 8 * hf;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + t * p.qr_stride_tok + h * p.qr_stride_head + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < kDLatent / 16; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qn + 16 * ks));
#pragma unroll
    for (int ks = 0; ks < kDRope / 16; ++ks)
      qf[kDLatent / 16 + ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 16 * ks));
  }

  f32x16_t o[2][4];  // O^T blocks: [row block][32-entry block of this wavefront's 128 entries]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[x][db][j] = 0.f;
  float m_ref0 = -INFINITY, m_ref1 = -INFINITY;  // per row block: reference max (log2 units)
  float l_part = 0.f;                       // this lane's share of its scoring row's softmax sum

  // Per-lane LDS byte offsets inside a tile buffer, recomputed per tile from
  // an opaque copy of the lane index (an XOR and a shift each).
  //   score operand (A of S^T = K Q^T): key qkey = 32kh + col; k-step ks
  //   reads latent piece 2ks + hf, stored at (2ks + hf) ^ swz(qkey) =
  //   2ks ^ sqh; rope k-step 32 + b reads rope piece 2b + hf of key qkey,
  //   stored at position (2b + hf) ^ (qkey % 8) = 2b ^ rsw of its row.
  //   value operand (A of O^T += V^T P^T, transposed reads): lane group row
  //   vr = (lane & 15) / 4 reads keys 32kh2 + 16c + 4hf + vr + 8x, latent
  //   entries d = 128w + 32db + 16g1 + 4(lane & 3) .. +3 (g1 = lane bit 4):
  //   piece 16w + 4db + vpl, vpl = 2g1 + (lane & 3) / 2, stored at
  //   16w + ((4db + vpl) ^ swz(vr + 8x)) = 16w + (vt ^ 4db ^ 8x), vt = vpl ^ swz(vr).
  struct LaneOffsets {
    int qbase, rbase, sqh, rsw, vbase, vt;
  };
  auto lane_offsets = [&](int ln) -> LaneOffsets {
    const int lhf = ln >> 5, lcol = ln & 31;
    const int qk = 32 * kh + lcol;
    const int vr = 4 * lhf + ((ln & 15) >> 2);
    LaneOffsets L;
    L.qbase = qk * kLatRow;
    L.rbase = kTileLat + qk * kRopeRow;
    L.rsw = lhf ^ (qk & 7);
    L.sqh = piece_swz(qk) ^ lhf;
    L.vbase = vr * kLatRow + 256 * wave + 8 * (ln & 1);
    L.vt = (2 * ((ln >> 4) & 1) + ((ln & 3) >> 1)) ^ piece_swz(vr);
    return L;
  };

  const float scale2 = p.sm_scale * kLog2e;
  const char* kvb = static_cast<const char*>(p.kv);
  const int64_t row_bytes = p.kv_stride * 2;

  // Slot of key `key` of this request. Keys past the split's end re-read the
  // last key (finite data whose probability is forced to zero), so every
  // load below is in bounds without a branch.
  auto slot_of = [&](int key) -> int {
    key = key < end ? key : end - 1;
    const int32_t* src = key < P ? p.kv_indices + ip0 + key : p.out_cache_loc + tb + (key - P);
    return *src;
  };
  // Visibility. The 32 rows of this wavefront's block belong to draft tokens
  // tok0 .. tok0+ntok-1 (one token when H is a multiple of 32). For each such
  // token, lane k (both halves alike) reads the mask byte of tile key
  // 32kh + k, and one ballot turns the 32 bytes into a bit mask; each lane
  // keeps its own token's. Bytes for four tokens are prefetched one tile
  // ahead (token indices clamped to the block's last); blocks spanning more
  // tokens (fewer than eight heads) read the rest when needed.
  const int rfirst = min(g * kRowsWG + rb * 32, R - 1);
  const int rlast = min(g * kRowsWG + rb * 32 + 31, R - 1);
  const int tok0 = rfirst / p.num_heads;
  const int ntok = rlast / p.num_heads - tok0 + 1;
  const int my_u = i - tok0;
  const uint8_t* mbase = p.mask + p.mask_indptr[b] + (int64_t)tok0 * N;
  uint8_t mnext[4];
  auto load_mask = [&](int p0) {
    int key = p0 + 32 * kh + col;
    key = key < end ? key : end - 1;
    mnext[0] = mbase[key];
    if (ntok > 1) {  // blocks of one token (at least 32 heads) need one byte
#pragma unroll
      for (int u = 1; u < 4; ++u) mnext[u] = mbase[(int64_t)min(u, ntok - 1) * N + key];
    }
  };
  auto visible_bits = [&](int p0) -> uint32_t {  // bit k: tile key 32kh + k visible to my row
    const int key = p0 + 32 * kh + col;
    const bool kok = key < end;
    if (ntok == 1) return (uint32_t)__ballot(kok && mnext[0] != 0);
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t bal = (uint32_t)__ballot(kok && mnext[u] != 0);
      mine = u == my_u ? bal : mine;
    }
    for (int u = 4; u < ntok; ++u) {
      const uint32_t bal = (uint32_t)__ballot(kok && mbase[(int64_t)u * N + (kok ? key : end - 1)] != 0);
      mine = u == my_u ? bal : mine;
    }
    return mine;
  };

  const int ntiles = (end - start + kKT - 1) / kKT;
  int slot_reg = slot_of(start + lane);
  auto row_address = [&](int slot, uint32_t& lo, uint32_t& hi) {
    const uint64_t a = (uint64_t)(uintptr_t)(kvb + (int64_t)slot * row_bytes);
    lo = (uint32_t)a;
    hi = (uint32_t)(a >> 32);
  };
  {
    uint32_t lo, hi;
    row_address(slot_reg, lo, hi);
#pragma unroll
    for (int u = 0; u < kKT / 4; ++u) stage_key(kb0, lo, hi, wave, lane, u);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      stage_rope(kb0, kvb + (int64_t)__shfl(slot_reg, 8 * (2 * wave + u) + (lane >> 3), 64) * row_bytes, wave, lane,
                 u);
  }
  load_mask(start);
  slot_reg = slot_of(start + kKT + lane);

  auto rescale = [&](f32x16_t (&ox)[4], float& mref, bool mine, float tmax) {
    const float m_new = fmaxf(mref, tmax);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref - m_new);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) ox[db][j] *= alpha;
    if (mine) l_part *= alpha;
    mref = m_new;
  };

  auto body = [&](int tile, const char* cur, char* nxt) {
    const int p0 = start + tile * kKT;
    tile_barrier();  // tile in LDS; every wavefront is done with the previous one
    const int ln = opaque(lane);
    const LaneOffsets L = lane_offsets(ln);
    // score register j of lane half hf holds tile key 32kh + 8(j/4) + 4hf + j%4
    const uint32_t vis = visible_bits(p0) >> (4 * hf);
    // Prefetch for the next tiles. On the last tile these re-read clamped,
    // valid rows into the idle buffer; nothing reads them.
    load_mask(p0 + kKT);
    const int slot_cur = slot_reg;
    slot_reg = slot_of(p0 + 2 * kKT + lane);
    uint32_t ra_lo, ra_hi;  // lane k: cache row address of the next tile's key k
    row_address(slot_cur, ra_lo, ra_hi);
    // slots of the next tile's rope keys 8(2 wave + u) + lane/8
    const int rslot0 = __shfl(slot_cur, 16 * wave + (ln >> 3), 64);
    const int rslot1 = __shfl(slot_cur, 16 * wave + 8 + (ln >> 3), 64);

    // ---- S^T = K Q^T: keys 32kh.. of the tile x the 32 rows of block rb.
    // The kRing k-steps ahead are read into a ring of operand registers so
    // each MFMA's LDS read was issued kRing MFMAs earlier. All eighteen of
    // the next tile's loads go here, one every second MFMA: the value product
    // below reads LDS harder, and loads issued there cost more.
    const uint32_t cur_lds = (uint32_t)(uintptr_t)TVMLA_LDS(const char, cur);
    auto kaddr = [&](int ks) -> uint32_t {
      return cur_lds + (ks < 32 ? L.qbase + (((2 * ks) ^ L.sqh) << 4) : L.rbase + (((2 * (ks - 32)) ^ L.rsw) << 4));
    };
    bf16x8_t ring[kRing];
#pragma unroll
    for (int x = 0; x < kRing; ++x) ring[x] = frag_read(kaddr(x));
    f32x16_t sacc;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      if (ks % 2 == 1 && ks < 32) stage_key(nxt, ra_lo, ra_hi, wave, ln, ks / 2);
      bf16x8_t& kf = ring[ks % kRing];
      wait_lgkm_tied(kf, min(kRing - 1, kQSteps - 1 - ks));
      if (ks == 0)
        TVMLA_MFMA_QK_FIRST(sacc, kf, qf[0]);
      else
        TVMLA_MFMA_QK(sacc, kf, qf[ks]);
      if (ks + kRing < kQSteps) kf = frag_read(kaddr(ks + kRing));
    }
    // Rope loads after the last operand wait, so the shuffles' wait is free.
    stage_rope(nxt, kvb + (int64_t)rslot0 * row_bytes, wave, ln, 0);
    stage_rope(nxt, kvb + (int64_t)rslot1 * row_bytes, wave, ln, 1);
    TVMLA_MFMA_DRAIN(sacc);

    // ---- O^T += V^T P^T for latent entries [128 wave, +128), both row blocks
    // (defined here: group 0's V^T reads are issued before the softmax).
    // Output register j of the score MFMA in lane half hf holds key
    // 8(j/4) + 4hf + j%4 of its 32; k-step c of the value product takes
    // registers 8c..8c+7, i.e. keys 16c + 8(j'/4) + 4hf + j'%4, j' = 0..7.
    // The transposed reads fetch V rows base..base+3 and base+8..base+11.
    // Four operand groups g = (kh2, c): eight transposed V^T reads (four
    // 32-entry blocks x two key quads) and the two P^T operands (one per row
    // block). Group g+1's reads are issued before group g's eight MFMAs.
    i16x4_t loA[4], hiA[4], loB[4], hiB[4];
    u32x4_t pbA[2], pbB[2];
    auto issue_v = [&](int grp, i16x4_t* lo, i16x4_t* hi) {
      const int kh2 = grp >> 1, c = grp & 1;
      const char* vb = cur + (32 * kh2 + 16 * c) * kLatRow + L.vbase;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        lo[db] = tr_read(vb + ((L.vt ^ (4 * db)) << 4));
        hi[db] = tr_read(vb + 8 * kLatRow + ((L.vt ^ (4 * db) ^ kSwzHi) << 4));
      }
    };
    auto issue_p = [&](int grp, u32x4_t* pb) {
      const int kh2 = grp >> 1, c = grp & 1;
#pragma unroll
      for (int x = 0; x < 2; ++x) pb[x] = lds_read128(&pex[((x + 2 * kh2) * 2 + c) * 64 + ln]);
    };
    auto issue = [&](int grp, i16x4_t* lo, i16x4_t* hi, u32x4_t* pb) {
      issue_v(grp, lo, hi);
      issue_p(grp, pb);
    };
    auto product = [&](const i16x4_t* lo, const i16x4_t* hi, const u32x4_t* pb) {
      bf16x8_t va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) va[db] = cat4(lo[db], hi[db]);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const bf16x8_t pbx = __builtin_bit_cast(bf16x8_t, pb[x]);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[x][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pbx, o[x][db], 0, 0, 0);
      }
    };
    issue_v(0, loA, hiA);

    // ---- row maxima over the whole 64-key tile (two wavefronts per row block).
    // Masked scores become -inf; when every score of the wavefront is
    // visible (the common case) the selects are skipped. sm_scale > 0, so the
    // maximum of the raw scores times scale2 is the maximum of the scaled
    // scores, exactly (rounding is monotonic).
    float sm[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[j] = sacc[j];
    constexpr uint32_t kVisAll = 0x0F0F0F0Fu;  // bits 8(j/4) + j%4, j = 0..15
    if (__ballot((vis & kVisAll) != kVisAll)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sm[j] = ((vis >> (8 * (j >> 2) + (j & 3))) & 1u) ? sm[j] : -INFINITY;
    }
    float tm = sm[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tm = fmaxf(tm, sm[j]);
    {
      // both lane halves hold the same rows: swap halves and combine
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
      tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale2;
    }
    // ---- probabilities of this wavefront's 32 keys x 32 rows, optimistically
    // against the current reference max: exp2(s * scale2 - m_ref), one fma
    // each (exp2(-inf) = 0 for masked keys). Only if some row of some
    // wavefront outgrew its reference by more than 2^8 (always on a split's
    // first visible tile) do all four take the exchange-and-rescale path
    // below and recompute; they all read the same flags, so they agree.
    bf16x8_t pf[2];
    float pj[16];
    auto probabilities = [&]() -> float {
      float mu = rb == 0 ? m_ref0 : m_ref1;
      mu = mu == -INFINITY ? 0.f : -mu;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        pj[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm[j], scale2, mu));
        pf[j >> 3][j & 7] = (__bf16)pj[j];
      }
      pex[(wave * 2 + 0) * 64 + lane] = as_u4(pf[0]);
      pex[(wave * 2 + 1) * 64 + lane] = as_u4(pf[1]);
      return ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7])) +
             (((pj[8] + pj[9]) + (pj[10] + pj[11])) + ((pj[12] + pj[13]) + (pj[14] + pj[15])));
    };
    const bool outgrown = __ballot(tm > (rb == 0 ? m_ref0 : m_ref1) + kRescaleLog2) != 0;
    float psum = probabilities();
    if (hf == 0) mex[wave * 32 + col] = tm;
    if (lane == 0) rescale_flag[wave] = outgrown;
    lds_barrier();

    // The flags are read along with group 0's operands. If any is set, all
    // four wavefronts exchange maxima, rescale, recompute and re-share their
    // probabilities, and re-read group 0 (its P^T operands were stale).
    u32x4_t fl = lds_read128(rescale_flag);
    issue_p(0, pbA);
    TVMLA_LDS_WAIT_F(loA, hiA, pbA, fl);
    if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3])) {
      // Every wavefront sees the same maxima and the same m_ref, so all four
      // rescale alike and keep identical references.
      const float tm0 = fmaxf(mex[col], mex[64 + col]);       // row block 0: wavefronts 0, 2
      const float tm1 = fmaxf(mex[32 + col], mex[96 + col]);  // row block 1: wavefronts 1, 3
      rescale(o[0], m_ref0, rb == 0, tm0);
      rescale(o[1], m_ref1, rb == 1, tm1);
      psum = probabilities();
      lds_barrier();
      issue(0, loA, hiA, pbA);
      TVMLA_LDS_WAIT(loA, hiA, pbA);
    }
    l_part += psum;
    // The scheduling barriers keep each group's MFMAs between the waits
    // (the compiler may otherwise hoist the next wait above them).
    issue(1, loB, hiB, pbB);
    TVMLA_PIN(loA, hiA, pbA);
    product(loA, hiA, pbA);
    __builtin_amdgcn_sched_barrier(0);
    TVMLA_LDS_WAIT(loB, hiB, pbB);
    issue(2, loA, hiA, pbA);
    TVMLA_PIN(loB, hiB, pbB);
    product(loB, hiB, pbB);
    __builtin_amdgcn_sched_barrier(0);
    TVMLA_LDS_WAIT(loA, hiA, pbA);
    issue(3, loB, hiB, pbB);
    TVMLA_PIN(loA, hiA, pbA);
    product(loA, hiA, pbA);
    __builtin_amdgcn_sched_barrier(0);
    TVMLA_LDS_WAIT(loB, hiB, pbB);
    product(loB, hiB, pbB);
  };

  for (int tile = 0; tile < ntiles; ++tile) {
    const bool odd = tile & 1;
    body(tile, odd ? kb1 : kb0, odd ? kb0 : kb1);
  }

  // The last tile's prefetch targeted the idle buffer; let it land before
  // the workgroup can exit and release its LDS.
  __builtin_amdgcn_s_waitcnt(0x0070);

  // ---- row sums: two wavefronts x two lane halves per row
  const float lt = l_part + __shfl_xor(l_part, 32, 64);
  lds_barrier();
  if (hf == 0) mex[wave * 32 + col] = lt;
  lds_barrier();
  const float lrow0 = mex[col] + mex[64 + col];
  const float lrow1 = mex[32 + col] + mex[96 + col];

  // ---- partial results: entries [128 wave, +128) of both row blocks
  auto write_block = [&](const f32x16_t (&ox)[4], float mref, float lrow, int x) {
    const int row = g * kRowsWG + 32 * x + col;
    if (row >= R) return;
    const size_t prow = ((size_t)b * p.nsplit + s) * Rw + row;
    uint16_t* dst = partial_bf16(p.o_part, prow) + 128 * wave + 4 * hf;  // bf16 in the slot's first 1 KB
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg)
        *reinterpret_cast<uint2*>(dst + 32 * db + 8 * jg) =
            pack_bf16x4(ox[db][4 * jg + 0] * inv, ox[db][4 * jg + 1] * inv, ox[db][4 * jg + 2] * inv,
                        ox[db][4 * jg + 3] * inv);
    if (wave == 0 && hf == 0) p.lse_part[prow] = lrow > 0.f ? (mref + log2f(lrow)) * kLn2 : -INFINITY;
  };
  write_block(o[0], m_ref0, lrow0, 0);
  write_block(o[1], m_ref1, lrow1, 1);
}

}  // namespace

hipError_t launch_split_mfma_bf16(const SplitParams& p, hipStream_t stream) {
  const int R = p.num_draft * p.num_heads;
  const int groups = (R + kRowsWG - 1) / kRowsWG;
  const int pairs = p.batch * p.nsplit;
  const int64_t blocks = (int64_t)8 * ((pairs + 7) / 8) * groups;
  SplitParams arg = p;
  int a_groups = groups, a_pairs = pairs;
  void* args[] = {&arg, &a_groups, &a_pairs};
  return hipLaunchKernel(reinterpret_cast<const void*>(&split_mfma_kernel), dim3((unsigned)blocks), dim3(256), args,
                         0, stream);
}

}  // namespace tvmla
