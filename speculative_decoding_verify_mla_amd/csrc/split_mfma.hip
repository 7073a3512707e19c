// bf16 MFMA split kernel for gfx950.
//
// Work unit: one workgroup = (request b, split s, group of 128 query rows).
// A request's rows are r = i*H + h (draft token i, head h); all of them share
// the request's keys, so one staged key tile feeds up to 128 rows at once --
// the reuse the sm_120 design reached with 8-head tiles ("The Plan
// Document", "The Design Reasoning", variant 3), here taken to 128 rows
// (64 heads x 2 tokens at the usual shape) because the contraction runs on
// the matrix cores.
//
// Per wavefront: 32 query rows. Scores are computed transposed,
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = key tile from LDS, B = the
// wavefront's 32 query rows, held in registers for the whole split), so the
// probabilities come out of the MFMA already in the layout the value product
// O^T += V^T P^T needs as its B operand; V^T (the 512 latent entries of the
// tile's keys, transposed) is the A operand, read from LDS. The output block
// O^T (512 x 32 fp32) stays in registers across the split.
//
// Schedule and indexing follow page 1, "The Design Emerges": split s of a
// request with N keys covers [s*chunk, min((s+1)*chunk, N)), chunk =
// ceil(N / nsplit), an empty split returns at once (first insight); a key's
// slot comes from kv_indices (prefix) or out_cache_loc (draft) (second);
// the mask byte is custom_mask[mask_indptr[b] + i*N + p] (third); P_b comes
// from kv_indptr (fourth). The online softmax (running max, running sum,
// rescaled accumulator; page 1, "Input Knowledge Required") rescales the
// accumulator only when a row's running max grows by more than 2^8, which
// keeps every probability below 256 and leaves the result unchanged.

#include "tvmla_internal.h"

namespace tvmla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kWaves = 4;
constexpr int kRowsWave = 32;
constexpr int kRowsWG = kWaves * kRowsWave;  // 128 query rows per workgroup
constexpr int kKT = 32;                       // keys per tile
constexpr int kKStr = kDKey + 8;              // staged key row: 584 bf16 (1168 B, skews LDS banks)
constexpr int kVTStr = kKT + 8;               // transposed latent entry: 40 bf16 (80 B)
constexpr int kQSteps = kDKey / 16;           // 36 k-steps of 16 over the key width
constexpr int kDBlocks = kDLatent / 32;       // 16 output blocks of 32 latent entries
constexpr float kRescaleLog2 = 8.f;           // lazy-rescale threshold (log2 units)

// Column of tile key k in the transposed latent tile. MFMA output register j
// of a lane in half `hf` holds key 8*(j/4) + 4*hf + j%4; value-product step c
// uses registers 8c..8c+7 as its B operand, i.e. keys
// 16c + 8*(j'/4) + 4*hf + j'%4 for j' = 0..7. Storing key k at column
// 16c + 8*hf + 4*(j'/4) + j'%4 puts each lane's eight keys side by side.
__device__ inline int vt_col(int k) {
  const int c = k >> 4, kp = k & 15;
  return (c << 4) + (((kp & 7) >> 2) << 3) + ((kp >> 3) << 2) + (kp & 3);
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_mfma_kernel(SplitParams p, int groups, int pairs) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKT * kKStr];
  __shared__ __attribute__((aligned(16))) uint16_t VT[kDLatent * kVTStr];

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
  const int b = pair / p.nsplit;
  const int s = pair - b * p.nsplit;

  const int R = p.num_draft * p.num_heads;
  const int ip0 = p.kv_indptr[b];
  const int P = p.kv_indptr[b + 1] - ip0;
  const int N = P + p.num_draft;
  int start, end;
  split_bounds(N, p.nsplit, p.min_chunk, s, start, end);
  if (start >= end) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5;   // which 8-wide half of each 16-wide k-step this lane feeds
  const int col = lane & 31;  // MFMA column = this lane's query row within the wavefront
  const int r = g * kRowsWG + wave * kRowsWave + col;
  const bool row_ok = r < R;
  // A row past the end computes on row R-1's data (its column of each MFMA
  // is independent of the others) and is never written.
  const int rr = row_ok ? r : R - 1;
  const int i = rr / p.num_heads;
  const int h = rr - i * p.num_heads;
  const int64_t tb = (int64_t)b * p.num_draft;  // first draft token of request b
  const int64_t t = tb + i;

  // Q^T fragments: query row `col`, key entries [16ks + 8hf, 16ks + 8hf + 8).
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

  f32x16_t o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_ref = -INFINITY;  // reference max (log2 units) the accumulator is scaled to
  float l_part = 0.f;       // this lane's share of the softmax sum

  const float scale2 = p.sm_scale * kLog2e;
  const uint8_t* mrow = p.mask + p.mask_indptr[b] + (int64_t)i * N;
  const uint16_t* kv = static_cast<const uint16_t*>(p.kv);

  for (int p0 = start; p0 < end; p0 += kKT) {
    __syncthreads();  // every wavefront is done with the previous tile

    // ---- stage the tile: lane -> key `col`, 16-byte pieces 2*(wave + 4q) + hf
    {
      // A key past the split's end re-reads the last key's row: finite data
      // whose probability is forced to zero below.
      const int key = min(p0 + col, end - 1);
      const int slot = key < P ? p.kv_indices[ip0 + key] : p.out_cache_loc[tb + (key - P)];
      const uint16_t* src = kv + (int64_t)slot * p.kv_stride;
      uint4 v[9];
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int piece = 2 * (wave + 4 * q) + hf;
        v[q] = *reinterpret_cast<const uint4*>(src + 8 * piece);
      }
      const int vc = vt_col(col);
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int piece = 2 * (wave + 4 * q) + hf;
        *reinterpret_cast<uint4*>(&Ks[col * kKStr + 8 * piece]) = v[q];
        if (piece < kDLatent / 8) {
          const uint32_t w4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            VT[(8 * piece + 2 * e) * kVTStr + vc] = (uint16_t)(w4[e] & 0xffffu);
            VT[(8 * piece + 2 * e + 1) * kVTStr + vc] = (uint16_t)(w4[e] >> 16);
          }
        }
      }
    }

    // ---- visibility of this lane's 16 keys: 8*(j/4) + 4*hf + j%4
    uint32_t vis = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = p0 + 8 * (j >> 2) + 4 * hf + (j & 3);
      const bool v = key < end && mrow[key] != 0;
      vis |= (uint32_t)v << j;
    }
    __syncthreads();  // the tile is in LDS

    // ---- S^T = K Q^T (32 keys x 32 rows), fp32 accumulation
    f32x16_t sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
    const uint16_t* kbase = Ks + col * kKStr + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kbase + 16 * ks);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
    }

    // ---- online softmax for row `col` (the two halves hold 16 keys each)
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sv[j] = ((vis >> j) & 1u) ? sacc[j] * scale2 : -INFINITY;
      tmax = fmaxf(tmax, sv[j]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__ballot(tmax > m_ref + kRescaleLog2)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      m_ref = m_new;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    bf16x8_t pf[2];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pj = exp2f(sv[j] - m_use);
      psum += pj;
      pf[j >> 3][j & 7] = (__bf16)pj;
    }
    l_part += psum;

    // ---- O^T += V^T P^T over the 512 latent entries
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
      const uint16_t* vrow = VT + (32 * db + col) * kVTStr + 8 * hf;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vrow + 16 * c);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], o[db], 0, 0, 0);
      }
    }
  }

  // ---- partial result: o / l and lse for this split
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (row_ok) {
    const size_t prow = ((size_t)b * p.nsplit + s) * R + r;
    float* dst = p.o_part + prow * kDLatent + 4 * hf;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        float4 v;
        v.x = o[db][4 * jg + 0] * inv;
        v.y = o[db][4 * jg + 1] * inv;
        v.z = o[db][4 * jg + 2] * inv;
        v.w = o[db][4 * jg + 3] * inv;
        *reinterpret_cast<float4*>(dst + 32 * db + 8 * jg) = v;
      }
    if (hf == 0) p.lse_part[prow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
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
