// bf16 MFMA split kernel for gfx950, row-owner form.
//
// Work unit: one workgroup = (request b, split s, group of 128 query rows).
// Wavefront w owns rows 32w .. 32w+31 of the group outright: it scores them
// against all 64 keys of every tile, keeps their softmax state, and accumulates
// their whole 512-entry output. Rows are r = i*H + h (draft token i, head h);
// every row of a request attends to the same keys, so one key tile staged in
// LDS feeds all 128 rows of the group ("The Plan Document", section "The Design
// Reasoning", variants 2 and 3: read the shared latent once, use it for many
// heads).
//
// LDS tile format: a 64-key tile is 8 groups of 8 keys. A key's cache row
// is 9 chunks of 128 bytes (8 latent, 1 rope; one cache line each), and
// chunk c of a group's 8 keys forms one 1 KB region, key by key, the
// key's 16-byte pieces XOR-swizzled inside its 128 bytes. Tiles are filled
// by direct global->LDS loads one tile ahead into a second buffer, one load
// per (group, chunk): 8 whole cache lines, each lane fetching from its own
// key's row, so no row address passes through scalar registers.
//
// Per tile, wavefront w:
//   scores   S^T = K Q^T for keys 0..31 and 32..63 of the tile (two 32x32
//            blocks, 36 k-steps each, v_mfma_f32_32x32x16_bf16; A = key rows
//            read from LDS, B = the wavefront's 32 queries, held in VGPRs for
//            the whole split);
//   softmax  each lane holds 32 of its row's 64 scores, so a row maximum --
//            taken only when a key block's probabilities outgrow the
//            reference (below) -- is a register maximum and one swap of lane
//            halves: no LDS exchange and no barrier. The probabilities,
//            rounded to bf16, already sit in the lanes and order the value
//            product takes as its B operand;
//   values   O^T += V^T P^T over all 512 latent entries (16 entry blocks x 4
//            key steps of 16), V^T read with the transposed LDS read
//            (ds_read_b64_tr_b16). O^T (512 x 32 fp32) lives in the 256
//            AGPRs for the whole split.
// Against the 64-row kernel this halves the staging loads and tile barriers
// per row and drops the probability exchange; in exchange every wavefront
// reads the whole tile from LDS (about 136 KB per wavefront per tile).
// Before the first tile and after the last one the tile buffers are free:
// the queries come in, and the output rows go out, through them, so that
// those memory accesses are whole rows rather than pieces of 32 rows.
//
// Split bounds, key slots, mask bytes and P_b follow "The Architecture of
// Capture Safety", "The Design Emerges" (chunk = ceil(N / nsplit), rounded up
// to whole 64-key tiles when the caller asks for that; empty split returns at
// once; slot from kv_indices for the prefix and out_cache_loc for draft keys;
// mask byte custom_mask[mask_indptr[b] + i*N + p]; P_b from kv_indptr). The
// online softmax ("The Architecture of Capture Safety", "Input Knowledge
// Required": running max, running sum, rescaled accumulator) keeps a per-row
// reference max and leaves the accumulator alone while the row's max stays
// within 2^fold_log2 of it (fold_log2 = 16: every probability stays below
// 65,536). When a row outgrows that, the wavefront folds: the accumulator goes
// to the rows' partial-result slots in the workspace (adding in what earlier
// folds left there, brought to the current reference), restarts from zero, and
// the reference moves up. The accumulator is never touched by vector
// instructions inside the tile loop -- only by MFMAs and by stores that read it
// straight from the AGPRs -- which is what keeps the compiler from moving it to
// VGPRs. The normalised result is the same for any threshold.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
#define TVMLA_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

constexpr int kRowsWG = 128;  // query rows per workgroup (4 wavefronts x 32)
constexpr int kKT = 64;       // keys per tile
constexpr int kGK = 8;                                 // keys per staging group
constexpr int kChunk = 128;                            // bytes of one key in one chunk (a cache line)
constexpr int kChunks = (2 * kDKey) / kChunk;          // 9 chunks per key: 8 latent, 1 rope
constexpr int kChunkBytes = kGK * kChunk;              // one chunk of a group's 8 keys: 1 KB
constexpr int kGroupBytes = kChunks * kChunkBytes;     // 9 KB per group
constexpr int kTileBytes = (kKT / kGK) * kGroupBytes;  // 73,728 bytes per tile buffer
constexpr int kRopeRow = 128;                          // bytes of one query row's rope part in LDS
constexpr int kQRow = 2 * kDLatent;                    // bytes of one query row's latent part (1 KB)
constexpr int kORow = kQRow + 8;                       // LDS stride of an output row in the epilogue
static_assert(2 * 32 * kORow <= kTileBytes, "two wavefronts' output rows fit in one tile buffer");
static_assert(2 * 32 * kQRow <= kTileBytes, "two wavefronts' query rows fit in one tile buffer");
constexpr int kQSteps = kDKey / 16;                    // 36 k-steps of 16 over the key width
constexpr int kSSteps = 2 * kQSteps;                   // score MFMAs per tile (two key blocks)
constexpr int kVSteps = 64;                            // value MFMAs per tile (16 entry blocks x 4 key steps)
constexpr int kSRing = 4;                              // score operand reads in flight
constexpr int kVRing = 4;                              // value steps in flight (two reads each)

// LDS reads a wavefront issues in the score phase of a tile: kSRing operand
// reads before step 0; after its MFMA, step m reads step m + kSRing's
// operand, at k-step 32 - kSRing also the four rope pieces of the queries,
// and in the last kVEarly steps the first value steps' operands (two reads
// each).
constexpr int kVEarly = 2;
constexpr int s_reads_issued(int m) {
  return (m + kSRing < kSSteps ? 1 : 0) + (m % kQSteps == 32 - kSRing ? kDRope / 16 : 0) + (m >= kSSteps - kVEarly ? 2 : 0);
}
// Reads issued after step r's operand read and before step n's MFMA.
constexpr int s_reads_after(int r, int n) {
  int c = 0;
  if (r < kSRing) {
    c = kSRing - 1 - r;
    for (int m = 0; m < n; ++m) c += s_reads_issued(m);
  } else {
    c = s_reads_issued(r - kSRing) - 1;
    for (int m = r - kSRing + 1; m < n; ++m) c += s_reads_issued(m);
  }
  return c;
}
static_assert(s_reads_after(3, 2) == 2 && s_reads_after(31, 30) == 6, "read counts");

// Piece swizzle: position j of key k's 128 bytes in a chunk holds piece
// j ^ xsw(k), xsw(k) = the three bits of (k % 16) / 2 in reverse order. A
// key's line lands on bank half k % 2 (128-byte lines, 256 bytes of banks),
// so the reads are conflict free when
//   score reads (16 lanes, 16 keys, one piece each): xsw over the 8 keys of
//     one parity among 16 consecutive keys is a permutation of 0..7;
//   score reads paired across lane halves (keys k < 8 read pieces j and
//     j ^ 1): xsw / 2 differs between the 4 keys of one parity;
//   transposed value reads (keys 2m and 2m + 2, m even, four pieces each):
//     xsw(2m) ^ xsw(2m + 2) = 4 puts them on disjoint position sets.
__host__ __device__ constexpr int xsw(int k) { return ((k & 2) << 1) | ((k & 4) >> 1) | ((k >> 3) & 1); }
// Piece swizzle of query row j (0..31) in LDS during the prologue: rows 0..7
// of 16 get even values 0..14, rows 8..15 odd ones.
__host__ __device__ constexpr int qsw(int j) { return ((j & 7) << 1) | ((j >> 3) & 1); }

template <int I>
struct Int {
  static constexpr int value = I;
};
// Compile-time loop: f(Int<i>) for i in [B, E); the index is a constant
// expression inside f, as the immediate operands of the inline asm need.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}

// Barrier at the top of a tile: this wavefront's loads into the tile have
// landed (vmcnt(0) expcnt(7) lgkmcnt(0) in the gfx9 encoding, via the
// builtin so the compiler knows every earlier load completed) and, after
// the barrier, so have everyone else's.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_barrier" ::: "memory");
}

// Workgroup barrier after this wavefront's LDS operations (not its global
// loads) have completed.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS operand reads through inline asm with an immediate offset. The
// compiler would treat its own LDS loads as possibly aliasing the in-flight
// direct-to-LDS loads and wait for all of them first; these reads are
// waited for explicitly (lgkmcnt) by the caller before use. LDS operations
// complete in order, so "at most n outstanding" after a read means the read
// is done once n later ones were issued.
template <int Off>
__device__ __forceinline__ bf16x8_t read_b128(uint32_t addr) {
  bf16x8_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(Off));
  return r;
}
template <int Off>
__device__ __forceinline__ i16x4_t read_tr(uint32_t addr) {
  i16x4_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(Off));
  return r;
}

// Score MFMA (accumulator in VGPRs, read by the softmax) and value MFMA
// (accumulator in AGPRs). Inline asm keeps the operands where they are; the
// compiler cannot see the hazards through it, so they are spelled out:
// TVMLA_S_DRAIN before vector code reads a score (24 wait states, twice
// what 8 passes need), and "s_nop 1" (2 wait states) in front of an MFMA
// whose operand may have just been written by a vector ALU instruction.
//
// The operand MFMAs wait for their LDS operands in the same statement
// ("s_waitcnt lgkmcnt(n)": at most n LDS operations of this wavefront still
// outstanding), once per pair of steps: the even step's MFMA waits for its
// own operand and the odd step's, and the odd step's MFMA (the _NW forms)
// issues without a wait. A separate wait statement would have to name the
// operand as an output, and the compiler then guards every MFMA behind it
// with a hazard nop as if a vector ALU instruction had just written the
// operand.
#define TVMLA_MFMA_S_FIRST(n, acc, a, q)                                                             \
  asm volatile("s_waitcnt lgkmcnt(%3)\n\ts_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) \
               : "v"(a), "v"(q), "n"(n))
#define TVMLA_MFMA_S(n, acc, a, q)                                                                            \
  asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(q), \
               "n"(n))
#define TVMLA_MFMA_S_NW(acc, a, q) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(q))
#define TVMLA_MFMA_O_NW(acc, a, p) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(p))
#define TVMLA_MFMA_O(n, acc, a, p)                                                                            \
  asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(p), \
               "n"(n))
#define TVMLA_MFMA_O_NOP(n, acc, a, p)                                                                        \
  asm volatile("s_waitcnt lgkmcnt(%3)\n\ts_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc)       \
               : "v"(a), "v"(p), "n"(n))
#define TVMLA_MFMA_ZERO(acc, z) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z))
#define TVMLA_S_DRAIN(s0, s1) asm volatile("s_nop 15\n\ts_nop 7" : "+v"(s0), "+v"(s1))
#define TVMLA_O_DRAIN(o)                                                                                          \
  asm volatile("s_nop 15\n\ts_nop 7"                                                                            \
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), \
                 "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),        \
                 "+a"(o[15]))

// Partial-result slot of a row: 512 fp32 latent entries. A lane's 16
// accumulator values of entry block db sit in four runs of 4 floats at
// stride 8 (entries 32db + 8jg + 4hf ..).
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
template <int J>
__device__ __forceinline__ f32x4_t quad(const f32x16_t& o) {
  return __builtin_shufflevector(o, o, 4 * J, 4 * J + 1, 4 * J + 2, 4 * J + 3);
}
// Plain stores of the accumulator quads: the compiler takes the data
// straight from the AGPRs. (Reading the accumulator with vector
// instructions inside the tile loop would make it keep the accumulator in
// VGPRs instead.)
__device__ __forceinline__ void store_block(float* slot, const f32x16_t& o) {
  *reinterpret_cast<f32x4_t*>(slot) = quad<0>(o);
  *reinterpret_cast<f32x4_t*>(slot + 8) = quad<1>(o);
  *reinterpret_cast<f32x4_t*>(slot + 16) = quad<2>(o);
  *reinterpret_cast<f32x4_t*>(slot + 24) = quad<3>(o);
}

#define TVMLA_MFMA_F32(acc, a, b) \
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x2_f32 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b))

// o^T += slot^T * diag(beta) for the wavefront's 32 rows, with fp32 MFMAs
// (32x32x2): A = two rows' slot entries per step (lane (k, i) holds entry
// 32db + i of row 2s + k), B = the matching two columns of diag(beta) (lane
// (k, j) holds beta_j when j = 2s + k). Each product adds one slot value
// times one beta, exactly as fp32 arithmetic does. `slot0` is the slot of
// the wavefront's row 0; rows at or past `rows` have no slot and add zero.
__device__ __forceinline__ void add_slots(f32x16_t (&o)[16], const float* slot0, int rows, float beta, int lane) {
  const int i = lane & 31, k = lane >> 5;
#pragma unroll
  for (int db = 0; db < 16; ++db) {
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const int q = 2 * s2 + k;
      const float a = q < rows ? __hip_atomic_load(slot0 + (size_t)q * kDLatent + 32 * db + i, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0.f;
      const float bb = i == q ? beta : 0.f;
      TVMLA_MFMA_F32(o[db], a, bb);
    }
    asm volatile("" ::: "memory");  // one block's loads at a time
  }
}

// max(a, b, c) in one instruction. fmaxf on values the compiler cannot
// prove canonical costs a canonicalizing max per operand besides the max.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// An opaque copy of a value: addresses derived from it are computed where
// they are used instead of being hoisted out of the tile loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ inline bf16x8_t cat4(i16x4_t lo, i16x4_t hi) {
  typedef __attribute__((ext_vector_type(8))) short i16x8_t;
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Direct-to-LDS staging load of chunk c of group G's 8 keys (1 KB). `a`
// is, in lane l, the address in its cache row's chunk 0 of the piece that
// lane stores: key 8G + l / 8, piece (l % 8) ^ xsw(key), at position l % 8
// of the key's 128 bytes. The chunk's 128c bytes are the load's immediate
// offset, which the hardware adds to the global and to the LDS address
// alike, so the LDS base given is 1024c - 128c past the group's (this spares
// a 64-bit address add per load). The loads of a tile go one at a time over
// the previous tile's score MFMAs. They are non-temporal (cache policy 2,
// `nt`): a cold call whose loads allocate in a MALL full of other dirty
// lines pays for their write-back (at 8 heads the cold split ran 104 us with
// ordinary loads, 66 us with these, the warm split 63 us either way).
template <int C>
__device__ __forceinline__ void stage_chunk(char* dst, const char* a, int G) {
  __builtin_amdgcn_global_load_lds(a, TVMLA_LDS(void, dst + G * kGroupBytes + C * (kChunkBytes - kChunk)), 16,
                                   kChunk * C, 2);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_rows_kernel(SplitParams p, int groups, int pairs) {
  __shared__ __attribute__((aligned(16))) char kb0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char kb1[kTileBytes];
  // the rope part of the 128 rows' queries (128 bytes per row, pieces
  // XOR-swizzled by the row): read for the four rope k-steps of each key
  // block instead of being held in registers for the whole split
  __shared__ __attribute__((aligned(16))) char qrope[kRowsWG * kRopeRow];

  // Workgroup ids reach the 8 XCDs round-robin (id % 8); every row group of
  // one (request, split) pair gets the same id % 8, so the pair's key rows
  // come from HBM once and are re-read from that XCD's L2.
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
  int64_t tb;
  request_tokens(p.qo_indptr, p.num_draft, b, Tb, tb);
  const int R = Tb * p.num_heads;
  if (g * kRowsWG >= R) return;
  const int ip0 = p.kv_indptr[b];
  const int P = p.kv_indptr[b + 1] - ip0;
  const int N = P + Tb;
  int start, end;
  split_bounds(N, p.nsplit, p.min_chunk, p.chunk_align, s, start, end);
  if (start >= end) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5;   // which 8-wide half of each 16-wide k-step this lane feeds
  const int col = lane & 31;  // MFMA column = query row within the wavefront

  // This lane's row. Rows past the end compute on row R-1's data (MFMA
  // columns are independent) and are never written.
  const int r = g * kRowsWG + 32 * wave + col;
  const int rr = r < R ? r : R - 1;
  const int i = rr / p.num_heads;
  const int h = rr - i * p.num_heads;
  const int64_t t = tb + i;

  bf16x8_t qf[kDLatent / 16];  // Q^T operands of the lane's row (loaded in the prologue below)

  f32x16_t o[16];  // O^T blocks: latent entries [32db, 32db + 32) x the 32 rows
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_ref = -INFINITY;  // the row's reference max (log2 units); both lane halves agree
  float l_part = 0.f;       // this lane's share of its row's softmax sum (since the last fold)
  float l_fold = 0.f;       // this lane's share of the folded sum (against m_slot)
  float m_slot = 0.f;       // the reference of the slot's folded sum
  bool folded = false;      // the partial-result slot holds a folded accumulator (wavefront-uniform)
  const bf16x8_t zero8 = {};
  // Partial-result row (valid when r < R). A workspace that fits in memory
  // has fewer than 2^32 rows of 2 KB. The 64-bit slot addresses are formed
  // where they are used (fold path, epilogue) from an opaque copy of it, not
  // kept in registers across the tile loop (which would spill them to
  // scratch, and a kernel that uses scratch pays several microseconds more
  // per launch).
  const uint32_t prow = (uint32_t)(((size_t)b * p.nsplit + s) * Rw + r);
  const int rows_valid = min(32, R - (g * kRowsWG + 32 * wave));

  const float scale2 = p.sm_scale * kLog2e;
  const float pthr = __builtin_amdgcn_exp2f(p.fold_log2);  // probability bound of the reference checks (inf for huge fold_log2)
  const char* kvb = static_cast<const char*>(p.kv);
  const int64_t row_bytes = p.kv_stride * 2;

  // Slot of key `key`; keys past the split's end re-read the last key
  // (finite data whose probability is forced to zero).
  auto slot_of = [&](int key) -> int {
    key = key < end ? key : end - 1;
    const int32_t* src = key < P ? p.kv_indices + ip0 + key : p.out_cache_loc + tb + (key - P);
    return *src;
  };
  // Visibility. The wavefront's 32 rows belong to draft tokens tok0 ..
  // tok0+ntok-1 (one token when H is a multiple of 32). Lane k reads the
  // mask byte of tile key k for each such token and a ballot turns the 64
  // bytes into a bit mask; each lane keeps its own token's. Bytes for four
  // tokens are prefetched a tile ahead; more tokens (fewer than eight heads)
  // are read when needed.
  const int rfirst = min(g * kRowsWG + 32 * wave, R - 1);
  const int rlast = min(g * kRowsWG + 32 * wave + 31, R - 1);
  const int tok0 = rfirst / p.num_heads;
  const int ntok = rlast / p.num_heads - tok0 + 1;
  const int my_u = i - tok0;
  const uint8_t* mbase = p.mask + p.mask_indptr[b] + (int64_t)tok0 * N;
  uint8_t mnext[4];
  auto load_mask = [&](int p0) {
    int key = p0 + lane;
    key = key < end ? key : end - 1;
    mnext[0] = mbase[key];
    if (ntok > 1) {
#pragma unroll
      for (int u = 1; u < 4; ++u) mnext[u] = mbase[(int64_t)min(u, ntok - 1) * N + key];
    }
  };
  auto visible_bits = [&](int p0) -> uint64_t {  // bit k: tile key k visible to my row
    const int key = p0 + lane;
    const bool kok = key < end;
    if (ntok == 1) return (uint64_t)__ballot(kok && mnext[0] != 0);
    uint64_t mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t bal = (uint64_t)__ballot(kok && mnext[u] != 0);
      mine = u == my_u ? bal : mine;
    }
    for (int u = 4; u < ntok; ++u) {
      const uint64_t bal = (uint64_t)__ballot(kok && mbase[(int64_t)u * N + (kok ? key : end - 1)] != 0);
      mine = u == my_u ? bal : mine;
    }
    return mine;
  };

  const int ntiles = (end - start + kKT - 1) / kKT;
  // Wavefront w stages groups 2w and 2w + 1 of each tile. gs0 / gs1: in lane
  // l, the slot of the key that lane serves in group 2w / 2w + 1 of the tile
  // being staged; `slot_reg` holds, in lane k, the slot of a tile's key k.
  int slot_reg;
  int gs0, gs1;
  // (ds_bpermute with the byte index of the source lane; the lane index is
  // recomputed here rather than held across the tile loop)
  auto group_slots = [&](int slots) {
    const int ln = opaque(lane);
    gs0 = __builtin_amdgcn_ds_bpermute(4 * (16 * wave + (ln >> 3)), slots);
    gs1 = __builtin_amdgcn_ds_bpermute(4 * (16 * wave + kGK + (ln >> 3)), slots);
  };
  auto chunk0 = [&](int slot, int u, int ln) -> const char* {
    return kvb + (int64_t)slot * row_bytes + 16 * ((ln & 7) ^ xsw(kGK * u + (ln >> 3)));
  };
  // ---- prologue. The first tile's group slots (loaded directly, no lane
  // exchange), the second tile's slots and the first tile's mask bytes go
  // out first; then the queries; then, once every wavefront holds its
  // queries, the first tile's staging.
  gs0 = slot_of(start + 16 * wave + (lane >> 3));
  gs1 = slot_of(start + 16 * wave + kGK + (lane >> 3));
  slot_reg = slot_of(start + kKT + lane);
  load_mask(start);

  // Q^T operands: the lane's row, key entries [16ks + 8hf, +8).
  //   latent (32 k-steps, kept in registers for the whole split): the
  //     wavefront's 32 rows pass through LDS -- the tile buffers, free until
  //     the first tile is staged, 32 KB per wavefront -- with one
  //     direct-to-LDS load per whole 1 KB row (8 full cache lines; loading
  //     the operand layout straight from memory takes 32 bytes of 32 rows
  //     per load, four times the memory requests), then 32 LDS reads in the
  //     operand layout. Piece P of row j sits at position P ^ qsw(j):
  //     conflict free for 16 lanes of one half (16 rows) and for 8 rows of
  //     both halves (even against odd positions).
  //   rope (4 k-steps, read from LDS at each tile's rope steps): rope piece
  //     2c + hf of local row x at position (2c + hf) ^ xsw(x % 16) of its
  //     128-byte row; the rows are 128 bytes apart like a chunk's keys, so
  //     the key swizzle keeps the reads conflict free.
  {
    char* qlat = (wave < 2 ? kb0 : kb1) + (wave & 1) * (32 * kQRow);
    const int x0 = g * kRowsWG + 32 * wave;  // the wavefront's first row (rows past R - 1 repeat row R - 1)
    int rj = min(x0, R - 1);
    int ij = rj / p.num_heads;
    int hj = rj - ij * p.num_heads;
    const uint16_t* qn0 = static_cast<const uint16_t*>(p.q_nope);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const char* row = reinterpret_cast<const char*>(qn0 + (tb + ij) * p.qn_stride_tok + (int64_t)hj * p.qn_stride_head);
      __builtin_amdgcn_global_load_lds(row + 16 * (lane ^ qsw(j)), TVMLA_LDS(void, qlat + j * kQRow), 16, 0, 0);
      if (x0 + j + 1 < R && ++hj == p.num_heads) {
        hj = 0;
        ++ij;
      }
    }
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + t * p.qr_stride_tok + h * p.qr_stride_head + 8 * hf;
    char* qrow = qrope + (32 * wave + col) * kRopeRow;
#pragma unroll
    for (int c = 0; c < kDRope / 16; ++c)
      *reinterpret_cast<uint4*>(qrow + (((2 * c + hf) ^ xsw(col & 15)) << 4)) =
          *reinterpret_cast<const uint4*>(qr + 16 * c);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's rows are in LDS
    const char* qmine = qlat + col * kQRow;
#pragma unroll
    for (int ks = 0; ks < kDLatent / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qmine + 16 * ((2 * ks + hf) ^ qsw(col)));
  }
  lds_barrier();  // every wavefront holds its queries: the tile buffers are free

  {
    const char* a0 = chunk0(gs0, 0, lane);
    const char* a1 = chunk0(gs1, 1, lane);
    static_for<0, kChunks>([&](auto c_) { stage_chunk<decltype(c_)::value>(kb0, a0, 2 * wave); });
    static_for<0, kChunks>([&](auto c_) { stage_chunk<decltype(c_)::value>(kb0, a1, 2 * wave + 1); });
  }
  group_slots(slot_reg);

  auto body = [&](int tile, const char* cur, char* nxt) {
    const int p0 = start + tile * kKT;
    const int ln = opaque(lane);
    const uint64_t vis = visible_bits(p0);
    load_mask(p0 + kKT);  // on the last tile these re-read clamped, valid bytes
    // next tile's staging address: chunk 0 of group 2w's rows (group 2w +
    // 1's is formed when its first load is due)
    const char* sa = chunk0(gs0, 0, ln);
    slot_reg = slot_of(p0 + 2 * kKT + lane);

    // ---- S^T = K Q^T, key block kb = n / 36, k-step ks = n % 36 (block 0's
    // chain, then block 1's). Score operand of lane (hf, col): key 32kb +
    // col (group 4kb + col / 8, line col % 8), piece 2ks + hf (rope for ks
    // >= 32): chunk ks / 4, position (2(ks % 4) + hf) ^ xsw(col). Four
    // address patterns (ks % 4) are registers; block and chunk are
    // immediate offsets.
    const uint32_t cur_lds = (uint32_t)(uintptr_t)TVMLA_LDS(const char, cur);
    const int lcol = ln & 31, lhf = ln >> 5;
    const int sx = xsw(lcol & 15) ^ lhf;
    const uint32_t sbase = cur_lds + (lcol >> 3) * kGroupBytes + (lcol & 7) * kChunk;
    const int rsw = lhf ^ xsw(lcol & 15);  // rope pieces of the queries (their own LDS rows)
    auto saddr = [&](auto n_) -> uint32_t {
      constexpr int n = decltype(n_)::value, ks = n % kQSteps;
      return sbase + (((2 * (ks % 4)) ^ sx) << 4);
    };
    auto sread = [&](auto n_) -> bf16x8_t {
      constexpr int n = decltype(n_)::value, kb = n / kQSteps, ks = n % kQSteps;
      constexpr int off = kb * (32 / kGK) * kGroupBytes + (ks / 4) * kChunkBytes;
      static_assert(off < 65536, "LDS offsets are 16-bit");
      return read_b128<off>(saddr(n_));
    };

    // ---- softmax pieces for key block h (keys 32h .. 32h+31 of the tile).
    // Score register j of block h in lane half hf holds key 32h + 8(j/4) +
    // 4hf + j%4. Masked scores become -inf (the whole wavefront seeing every
    // key of the tile -- the common case -- skips the selects). sm_scale > 0,
    // so the maximum of the raw scores times scale2 is the maximum of the
    // scaled scores exactly. Probabilities are taken against the current
    // reference m_ref (exp2(s * scale2 - m_ref), one fma each; exp2(-inf) =
    // 0): valid unless the block's max outgrows the reference, which the
    // caller checks before using them.
    const uint64_t vh = vis >> (4 * hf);
    constexpr uint32_t kVisAll = 0x0F0F0F0Fu;  // bits 8(j/4) + j%4, j = 0..15
    const bool allvis = __ballot((((uint32_t)vh & kVisAll) != kVisAll) || (((uint32_t)(vh >> 32) & kVisAll) != kVisAll)) == 0;
    float sm[2][16], tmx[2], psum[2];
    bf16x8_t pf[4];  // P^T operand of key step q = 2h + c
    auto mask_block = [&](int h) {
      if (!allvis) {
        const uint32_t v = (uint32_t)(vh >> (32 * h));
#pragma unroll
        for (int j = 0; j < 16; ++j) sm[h][j] = ((v >> (8 * (j >> 2) + (j & 3))) & 1u) ? sm[h][j] : -INFINITY;
      }
    };
    // The side work between MFMAs is issued in order with them: an
    // instruction that waits on the one before it (an exp on its fma, an add
    // on its exp) holds back the next MFMA as well. So each probability is
    // three stages one gap apart.
    // Probability j of block h against mu = -m_ref (0 while m_ref = -inf):
    // F (the fma into pt[j]), E (exp2 in place), S (the running sum, and for
    // odd j the pair packed into the P^T operand). prob_stage(h, k, mu) is
    // step k of the pipeline: S(k-2), E(k-1), F(k); steps 0..17 cover j =
    // 0..15, each stage one step after the one it needs. The sum runs over
    // j = 0..15 in order as before. The steps go into two of every three
    // MFMA gaps (27 gaps), which leaves the exp2 (a quarter-rate
    // instruction) more room beside the MFMAs than three stages every gap.
    float pt[16];
    auto prob_f = [&](int h, int j, float mu) { pt[j] = __builtin_fmaf(sm[h][j], scale2, mu); };
    auto prob_e = [&](int j) { pt[j] = __builtin_amdgcn_exp2f(pt[j]); };
    auto prob_s = [&](int h, int j) {
      psum[h] = j == 0 ? pt[j] : psum[h] + pt[j];
      if (j & 1) {
        pf[2 * h + (j >> 3)][(j & 7) - 1] = (__bf16)pt[j - 1];
        pf[2 * h + (j >> 3)][j & 7] = (__bf16)pt[j];
      }
    };
    auto prob_stage = [&](int h, int k, float mu) {
      if (k >= 2 && k < 18) prob_s(h, k - 2);
      if (k >= 1 && k < 17) prob_e(k - 1);
      if (k < 16) prob_f(h, k, mu);
    };
    constexpr int kProbGaps = 18;
    auto probs_block = [&](int h, float mu) {
#pragma unroll
      for (int k = 0; k < kProbGaps; ++k) prob_stage(h, k, mu);
    };
    // The block's maximum per row, scaled: a row's 32 keys sit in lanes col
    // and col + 32. Only the reference checks below need it.
    auto max_block = [&](int h) {
      float mx = sm[h][0];
#pragma unroll
      for (int j = 1; j < 15; j += 2) mx = max3(mx, sm[h][j], sm[h][j + 1]);
      mx = fmaxf(mx, sm[h][15]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      tmx[h] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale2;
    };
    const float mu0 = m_ref == -INFINITY ? 0.f : -m_ref;
    // Keeps block h's probabilities and sum where they are computed (a
    // reference check below recomputes them when the reference moves).
    auto pin_probs = [&](int h) { asm volatile("" ::"v"(pf[2 * h]), "v"(pf[2 * h + 1]), "v"(psum[h])); };

    // ---- value product O^T += V^T P^T, step n: key step q = n / 16 (keys
    // 16q ..), entry block db = n % 16. Key step q = 2h + c takes score
    // registers 8c .. 8c+7 of block h, i.e. keys 16q + 8(m/4) + 4hf + m%4
    // (m = 0..7), so the V^T operand holds V rows 16q + vr (lo) and 16q +
    // vr + 8 (hi), vr = 4hf + (lane & 15) / 4: the lane reads latent entries
    // 32db + 16 g1 + 4(lane & 3) .. +3 (g1 = lane bit 4), i.e. piece 4db +
    // vpl (vpl = 2 g1 + (lane & 3) / 2), byte 8(lane & 1) -- of key 16q + vr
    // + 8x: group 2q + x, line vr, chunk db / 2, position (4(db % 2) + vpl)
    // ^ xsw(vr + 8x). Four address patterns (x, db % 2) are registers.
    const int vr = 4 * lhf + ((ln & 15) >> 2);
    const int vpl = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
    const uint32_t vbase = cur_lds + vr * kChunk + 8 * (ln & 1);
    auto vaddr = [&](int x, int d2) -> uint32_t {
      return vbase + x * kGroupBytes + (((4 * d2 + vpl) ^ xsw(vr + kGK * x)) << 4);
    };
    i16x4_t vlo[kVRing], vhi[kVRing];
    auto vread = [&](auto n_) {
      constexpr int n = decltype(n_)::value, q = n / 16, db = n % 16;
      constexpr int off = 2 * q * kGroupBytes + (db / 2) * kChunkBytes;
      static_assert(off < 65536, "LDS offsets are 16-bit");
      vlo[n % kVRing] = read_tr<off>(vaddr(0, db % 2));
      vhi[n % kVRing] = read_tr<off>(vaddr(1, db % 2));
    };
    // value steps [B, E); `side(i)` runs between steps (i = step - B)
    auto pv_steps = [&](auto b_, auto e_, auto&& side) {
      constexpr int B = decltype(b_)::value, E = decltype(e_)::value;
      static_for<B, E>([&](auto n_) {
        constexpr int n = decltype(n_)::value, q = n / 16, db = n % 16;
        // even steps wait for this step's and the next step's operands: at
        // most the reads of the steps after n + 1 stay outstanding
        constexpr int ahead = 2 * (kVSteps - 2 - n < kVRing - 2 ? kVSteps - 2 - n : kVRing - 2);
        static_assert(kVSteps % 2 == 0 && kVRing >= 2, "value steps wait in pairs");
        if constexpr (db == 0)  // pf[q] is vector-ALU output: two wait states before an MFMA reads it
          TVMLA_MFMA_O_NOP(ahead, o[db], cat4(vlo[n % kVRing], vhi[n % kVRing]), pf[q]);
        else if constexpr (n % 2 == 0)
          TVMLA_MFMA_O(ahead, o[db], cat4(vlo[n % kVRing], vhi[n % kVRing]), pf[q]);
        else
          TVMLA_MFMA_O_NW(o[db], cat4(vlo[n % kVRing], vhi[n % kVRing]), pf[q]);
        if constexpr (n + kVRing < kVSteps) vread(Int<n + kVRing>{});
        side(Int<n - B>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- scores. Block 0's softmax pieces ride along block 1's MFMAs
    // (from two MFMAs after block 0's last, when its results are written).
    // The next tile's 18 staging loads (two groups x 9 chunks) go one per
    // four MFMAs.
    // The rope part of the queries is read from LDS four k-steps before the
    // block's rope steps, right after that step's operand read, so the
    // operand wait of the first rope step covers it as well. The last
    // kVEarly steps read the first kVEarly value steps' operands, which so
    // arrive under the last score MFMAs (the rest of the value ring is read
    // after block 0's reference check: held across it, more of the ring
    // would not fit the registers).
    const uint32_t qrbase = (uint32_t)(uintptr_t)TVMLA_LDS(const char, qrope) + (32 * wave + lcol) * kRopeRow;
    bf16x8_t ring[kSRing], qrf[kDRope / 16];
    static_for<0, kSRing>([&](auto x_) { ring[decltype(x_)::value] = sread(x_); });
    f32x16_t sacc[2];
    static_for<0, kSSteps>([&](auto n_) {
      constexpr int n = decltype(n_)::value, kb = n / kQSteps, ks = n % kQSteps;
      if constexpr (n % 4 == 1 && n / 4 < 2 * kChunks) {
        constexpr int j = n / 4;
        if constexpr (j == kChunks) sa = chunk0(opaque(gs1), 1, ln);
        stage_chunk<j % kChunks>(nxt, sa, 2 * wave + j / kChunks);
      }
      bf16x8_t& kf = ring[n % kSRing];
      // even steps wait for this step's and the next step's operands: at
      // most the LDS reads issued after step n + 1's operand read stay
      // outstanding (LDS reads complete in order)
      constexpr int ahead = s_reads_after(n + 1, n);
      static_assert(kQSteps % 2 == 0, "score steps wait in pairs within each block");
      const bf16x8_t& qop = ks < 32 ? qf[ks < 32 ? ks : 0] : qrf[ks < 32 ? 0 : ks - 32];
      if constexpr (ks == 0)
        TVMLA_MFMA_S_FIRST(ahead, sacc[kb], kf, qf[0]);
      else if constexpr (n % 2 == 0)
        TVMLA_MFMA_S(ahead, sacc[kb], kf, qop);
      else
        TVMLA_MFMA_S_NW(sacc[kb], kf, qop);
      if constexpr (n + kSRing < kSSteps) kf = sread(Int<n + kSRing>{});
      if constexpr (n >= kSSteps - kVEarly) vread(Int<n - (kSSteps - kVEarly)>{});
      static_assert(kSRing == 4, "the rope operand reads assume four operand reads in flight");
      if constexpr (ks == 32 - kSRing) {
        static_for<0, kDRope / 16>([&](auto c_) {
          constexpr int c = decltype(c_)::value;
          qrf[c] = read_b128<0>(qrbase + (((2 * c) ^ rsw) << 4));
        });
      }
      constexpr int i = n - (kQSteps + 2);  // block 0's pieces, about one MFMA's worth each
      if constexpr (i == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sm[0][j] = sacc[0][j];
        mask_block(0);
      }
      constexpr int k0 = i - 1;        // gap of block 0's probability pipeline
      constexpr int g0 = k0 - k0 / 3;  // pipeline step of this gap (every third gap empty)
      if constexpr (k0 >= 0 && k0 % 3 != 2 && g0 < kProbGaps) prob_stage(0, g0, mu0);
      static_assert(kQSteps + 2 + 1 + (3 * kProbGaps) / 2 <= kSSteps, "block 0's softmax must fit under block 1's MFMAs");
      // Keep them here: the reference check below recomputes them when the
      // reference moves, and the compiler would otherwise sink them into the
      // other branch, after the last score MFMA.
      if constexpr (k0 >= 0 && k0 % 3 != 2 && g0 == kProbGaps - 1) pin_probs(0);
      __builtin_amdgcn_sched_barrier(0);
    });

    // Reference max. A row whose max exceeds its reference by more than
    // fold_log2 takes a new reference: at once if it has accumulated nothing
    // yet (reference -inf); otherwise the wavefront first folds its
    // accumulator into the rows' partial-result slots and restarts it from
    // zero (the accumulator is only ever touched by MFMAs and by memory
    // instructions that read it straight from the AGPRs, which keeps it
    // there).
    auto fold = [&]() {
      // slot = O + slot * 2^(m_slot - m_ref), against m_ref (a row with
      // nothing accumulated at the last fold has m_slot = -inf and a zero slot)
      const uint32_t pr = opaque(prow);
      float* fold_dst = p.o_part + (size_t)pr * kDLatent + 4 * opaque(hf);
      const float* slot0 = p.o_part + (size_t)(pr - col) * kDLatent;  // slot of the wavefront's row 0
      const float beta = m_slot == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_slot - m_ref);
      TVMLA_O_DRAIN(o);
      if (folded) add_slots(o, slot0, rows_valid, beta, ln);
      TVMLA_O_DRAIN(o);
      if (r < R) {
#pragma unroll
        for (int db = 0; db < 16; ++db) store_block(fold_dst + 32 * db, o[db]);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      l_fold = folded ? l_fold * beta + l_part : l_part;
      l_part = 0.f;
      m_slot = m_ref;
      folded = true;
#pragma unroll
      for (int db = 0; db < 16; ++db) TVMLA_MFMA_ZERO(o[db], zero8);
    };
    // Reference checks, one per key block. A block's probabilities are taken
    // against the current reference; the reference has to move only when
    // one of them exceeds 2^fold_log2 (the block's max outgrew the
    // reference by more than fold_log2) or when a row with no reference yet
    // (-inf) sees a key. A probability above the bound puts its lane's
    // partial sum above it too (and an overflow makes the sum inf), so the
    // lane sums decide: a wavefront with no such lane -- the common case --
    // goes on with no maximum computed. Otherwise it computes the block's
    // maximum and moves the reference as online softmax does: rows whose max
    // outgrew the reference take it as their new one -- after the wavefront
    // folds its accumulator into the rows' partial-result slots if they have
    // accumulated something -- and the block's probabilities are redone.
    // (Once set from data, a reference is some key's score, whose probability
    // 1 keeps the row's sum from underflowing.)
    auto vis_any = [&](int h) { return allvis || ((((uint32_t)(vh >> (32 * h))) & kVisAll) != 0u); };
    auto check_block = [&](int h) {
      const bool need = (m_ref == -INFINITY && vis_any(h)) || psum[h] >= pthr;
      if (__ballot(need)) {
        max_block(h);
        const bool grow = tmx[h] > m_ref + p.fold_log2;
        if (__ballot(grow && m_ref != -INFINITY)) fold();
        m_ref = grow ? tmx[h] : m_ref;
        probs_block(h, m_ref == -INFINITY ? 0.f : -m_ref);
      }
    };
    check_block(0);
    const float mu1 = m_ref == -INFINITY ? 0.f : -m_ref;
    static_for<kVEarly, kVRing>([&](auto x_) { vread(x_); });

    // ---- value steps of block 0 with block 1's probabilities computed
    // alongside (against the reference block 0 left), block 1's check (a
    // fold there takes block 0's products and sum with it), then block 1's
    // value steps
    pv_steps(Int<0>{}, Int<32>{}, [&](auto i_) {
      constexpr int i = decltype(i_)::value;
      if constexpr (i == 0) {
        asm volatile("s_nop 15\n\ts_nop 7" : "+v"(sacc[1]));  // block 1's last MFMA results are written
#pragma unroll
        for (int j = 0; j < 16; ++j) sm[1][j] = sacc[1][j];
        mask_block(1);
      }
      constexpr int k1 = i - 1, g1 = k1 - k1 / 3;
      if constexpr (k1 >= 0 && k1 % 3 != 2 && g1 < kProbGaps) prob_stage(1, g1, mu1);
      if constexpr (k1 >= 0 && k1 % 3 != 2 && g1 == kProbGaps - 1) pin_probs(1);
    });
    l_part += psum[0];
    check_block(1);
    l_part += psum[1];
    pv_steps(Int<32>{}, Int<64>{}, [](auto) {});
    group_slots(slot_reg);  // for the tile after next, staged by the next tile
  };
  for (int tile = 0; tile < ntiles; ++tile) {
    tile_barrier();  // tile in LDS; every wavefront is done with the previous one
    const bool odd = tile & 1;
    body(tile, odd ? kb1 : kb0, odd ? kb0 : kb1);
  }
  // The last tile's prefetch targeted the idle buffer; let it land before
  // the workgroup exits and releases its LDS.
  __builtin_amdgcn_s_waitcnt(0x0070);
  TVMLA_O_DRAIN(o);

  // The folded part (against m_slot) joins the accumulator (against m_ref).
  const uint32_t pr = opaque(prow);
  const float beta = folded && m_slot != -INFINITY ? __builtin_amdgcn_exp2f(m_slot - m_ref) : 0.f;
  if (folded) {
    add_slots(o, p.o_part + (size_t)(pr - col) * kDLatent, rows_valid, beta, lane);
    TVMLA_O_DRAIN(o);
  }
  const float lsum = l_fold * beta + l_part;
  // the row's two lane halves: lane k < 32 adds lane k + 32's share, lane k + 32 lane k's
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
  const float l = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (hf == 0 && r < R) p.lse_part[pr] = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;

  // The rows' normalised outputs as bf16 (each row slot's first 1 KB) go
  // out as two stores of 512 contiguous bytes per row: written straight
  // from the accumulator layout, a store would take 16 bytes of each of 32
  // rows, eight times the memory requests. So they pass through LDS: once
  // every wavefront is past its last tile the tile buffers are free, and the
  // wavefront's 32 rows take 33 KB, row j at j * 1032 bytes with its 8-byte
  // unit u (entries 4u .. 4u+3) at 8u. The 129-unit row stride puts unit u
  // of the 32 rows on 32 distinct bank pairs (row j's on pair (j + u) mod
  // 32), and a row's read-back (lane l: units l and l + 64) covers
  // consecutive units.
  lds_barrier();
  char* obuf = (wave < 2 ? kb0 : kb1) + (wave & 1) * (32 * kORow);
  {
    char* orow = obuf + col * kORow + 8 * hf;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg)
        *reinterpret_cast<uint2*>(orow + 64 * db + 16 * jg) =
            pack_bf16x4(o[db][4 * jg + 0] * inv, o[db][4 * jg + 1] * inv, o[db][4 * jg + 2] * inv,
                        o[db][4 * jg + 3] * inv);
  }
  const uint32_t pr0 = pr - col;  // the wavefront's first partial-result row
  for (int j = 0; j < rows_valid; ++j) {
    const char* src = obuf + j * kORow + 8 * lane;
    const uint2 v0 = *reinterpret_cast<const uint2*>(src);
    const uint2 v1 = *reinterpret_cast<const uint2*>(src + 512);
    uint16_t* dst = partial_bf16(p.o_part, pr0 + j) + 4 * lane;
    *reinterpret_cast<uint2*>(dst) = v0;
    *reinterpret_cast<uint2*>(dst + 256) = v1;
  }
}

}  // namespace

hipError_t launch_split_rows_bf16(const SplitParams& p, hipStream_t stream) {
  const int R = p.num_draft * p.num_heads;
  const int groups = (R + kRowsWG - 1) / kRowsWG;
  const int pairs = p.batch * p.nsplit;
  const int64_t blocks = (int64_t)8 * ((pairs + 7) / 8) * groups;
  SplitParams arg = p;
  int a_groups = groups, a_pairs = pairs;
  void* args[] = {&arg, &a_groups, &a_pairs};
  return hipLaunchKernel(reinterpret_cast<const void*>(&split_rows_kernel), dim3((unsigned)blocks), dim3(256), args,
                         0, stream);
}

}  // namespace tvmla
