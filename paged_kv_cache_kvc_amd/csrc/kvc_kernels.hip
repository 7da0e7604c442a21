// HIP kernels of the two-stream paged KV-cache attention for gfx950 (MI355X).
//
//   append_kernel  - writes one frame's K/V rows of one block into its patch
//                    page and its special-stream slots ([p5] "How Paged KV
//                    Cache Attention Achieves Stable Inference in
//                    Ling-Bot-Map" §Frame Appending Without Dispatch Overhead).
//   attn_kernel    - paged prefill attention of the frame's queries over the
//                    visible pages, o = softmax(q K^T / sqrt(D)) V, with bf16
//                    MFMA and a float32 online softmax; optionally over one KV
//                    split, writing a normalised partial output and its
//                    log-sum-exp ([p2] "How LingBot-Map Uses FlashInfer KV
//                    Cache for Streaming 3D Reconstruction" §Attention Kernel
//                    Execution; [p5] §Kernel Dispatch and Sequence Lengths).
//   merge_kernel   - combines the KV splits of a row in fixed split order.
//   attn_f32_kernel - paged attention on float32 pools (float32 MFMA,
//                    probabilities not rounded), one wave per 16 queries.
//   rope_kernel    - rotary position embedding of the step's query rows with
//                    caller tables ([p2] §3D RoPE Position Encoding); the
//                    key rows are turned inside append_kernel on their way to
//                    the pool.
//
// Layouts: pool [pages, 2, page_size, H, D] bf16 (NHD inside a page, [p1]
// "How FlashInfer KV Cache Attention Accelerates Streaming 3D Reconstruction
// Over SDPA" §Paged KV Cache Memory Layout); q, o [rows, H, D] bf16.
//
// Attention work item = (stream, head, KV split, query group).  A work-group
// of 4 waves streams its split's KV through a ring of LDS stages (64 slots of
// one page each) with direct global-to-LDS loads.  K and V stay row-major in
// LDS; V is read as the transposed MFMA operand with ds_read_b64_tr_b16.  The
// scores are computed transposed, S^T = K Q^T (16x16x32 bf16 MFMA, kv on rows,
// queries on columns), so each lane's accumulators belong to one query column:
// the softmax column max needs only two cross-lane steps, and the
// probabilities feed the P.V MFMA (O^T = V^T P^T) straight from registers.
// Rule kept throughout: an MFMA result is never read by a vector instruction
// right after its MFMA is issued; every consumer is one pipelined tile later.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kvc.h"
#include "kvc_device.h"
#include "kvc_kernels.h"

namespace kvc {

namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// rotary position embedding
// ---------------------------------------------------------------------------
// Positions are applied to q and k before the cache, so attention needs no
// position lookup ([p2] "How LingBot-Map Uses FlashInfer KV Cache for
// Streaming 3D Reconstruction" §3D RoPE Position Encoding and its FAQ on
// temporal information).  The pages give no frequencies: the caller passes
// float32 tables cos, sin [rows, D/2], entry (t, i) turning elements
// (2i, 2i+1) of every head of row t as (a, b) -> (a c - b s, a s + b c).
//
// The rotation is computed in float64.  A product of a 16-bit element and a
// float32 table value has at most 35 significant bits, so both products are
// exact there and the only roundings are the sum's (to float64) and the final
// one to the element type, done as a single rounding to nearest even: the
// value is first narrowed to float32 toward zero with the discarded bits
// kept as a sticky last bit (round to odd, 24 >= 11 + 2 bits), which a
// second rounding to 8 or 11 bits cannot tell from the float64 value.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float t = __double2float_rz(x);
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, t) | ((double)t != x ? 1u : 0u));
}

template <int E>
__device__ __forceinline__ double elem_to_f64(uint32_t w, int half);
template <>
__device__ __forceinline__ double elem_to_f64<0>(uint32_t w, int half) {
  return (double)__builtin_bit_cast(float, half ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ double elem_to_f64<1>(uint32_t w, int half) {
  return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(half ? (w >> 16) : (w & 0xFFFFu)));
}
// float32: one element per word (`half` unused)
template <>
__device__ __forceinline__ double elem_to_f64<2>(uint32_t w, int half) {
  return (double)__builtin_bit_cast(float, w);
}

template <int E>
__device__ __forceinline__ uint32_t f64_to_elem(double x);
template <>
__device__ __forceinline__ uint32_t f64_to_elem<0>(double x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f64_to_f32_odd(x));
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <>
__device__ __forceinline__ uint32_t f64_to_elem<1>(double x) {
  return __builtin_bit_cast(uint16_t, (_Float16)f64_to_f32_odd(x));
}
template <>
__device__ __forceinline__ uint32_t f64_to_elem<2>(double x) {
  return __builtin_bit_cast(uint32_t, (float)x);   // one rounding to nearest even
}

// One 16-byte chunk: four (even, odd) pairs of 16-bit elements, each 32-bit
// word one pair; or, for float32 (E = 2), two pairs in words (0, 1), (2, 3).
// c and s hold the chunk's pairs' table entries (two used for float32).
template <int E>
__device__ __forceinline__ u32x4 rope_chunk(const u32x4& x, const f32x4& c, const f32x4& s) {
  u32x4 y;
  if constexpr (E == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const double a = elem_to_f64<E>(x[2 * j], 0), b = elem_to_f64<E>(x[2 * j + 1], 0);
      const double cj = (double)c[j], sj = (double)s[j];
      y[2 * j] = f64_to_elem<E>(a * cj - b * sj);
      y[2 * j + 1] = f64_to_elem<E>(a * sj + b * cj);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = elem_to_f64<E>(x[j], 0), b = elem_to_f64<E>(x[j], 1);
      const double cj = (double)c[j], sj = (double)s[j];
      y[j] = f64_to_elem<E>(a * cj - b * sj) | (f64_to_elem<E>(a * sj + b * cj) << 16);
    }
  }
  return y;
}

// Table entries of the pairs of 16-byte chunk i of a row (elements 16 / elem
// bytes per chunk): four for 16-bit elements, two for float32.
template <int E>
__device__ __forceinline__ void rope_entries(const float* cos_row, const float* sin_row, uint32_t i, int head_dim,
                                             f32x4& c, f32x4& s) {
  constexpr uint32_t EPC = E == 2 ? 4 : 8;   // elements per chunk
  const uint32_t pair0 = ((i * EPC) & (uint32_t)(head_dim - 1)) >> 1;
  if constexpr (E == 2) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 c2 = *reinterpret_cast<const f32x2*>(cos_row + pair0);
    const f32x2 s2 = *reinterpret_cast<const f32x2*>(sin_row + pair0);
    c = f32x4{c2[0], c2[1], 0.f, 0.f};
    s = f32x4{s2[0], s2[1], 0.f, 0.f};
  } else {
    c = *reinterpret_cast<const f32x4*>(cos_row + pair0);
    s = *reinterpret_cast<const f32x4*>(sin_row + pair0);
  }
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
// ROPE: -1 copies K as it is; 0 (bf16) or 1 (f16) turns it by row r of the
// tables on the way.
template <int ROPE>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int r = blockIdx.x;
  const int off = p.special_row_offset;
  int page, slot;
  if (r >= off && r < off + p.n_special) {
    const int pos = p.sp_slot0 + (r - off);
    const int idx = pos / p.page_size;
    page = p.sp_pages[0];
#pragma unroll
    for (int i = 1; i < KVC_MAX_APPEND_SPECIAL_PAGES; ++i)
      if (i == idx) page = p.sp_pages[i];
    slot = pos - idx * p.page_size;
  } else {
    page = p.patch_page;
    slot = r < off ? r : r - p.n_special;
  }
  const size_t row_bytes = (size_t)p.row_elems * p.elem_bytes;
  const int chunks = (int)(row_bytes >> 4);   // 16-byte chunks per row; H*D is a multiple of 32
  const u32x4* sk = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.k) + (size_t)r * row_bytes);
  const u32x4* sv = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.v) + (size_t)r * row_bytes);
  uint8_t* pool = static_cast<uint8_t*>(p.pool);
  u32x4* dk = reinterpret_cast<u32x4*>(pool + (((size_t)page * 2 + 0) * p.page_size + slot) * row_bytes);
  u32x4* dv = reinterpret_cast<u32x4*>(pool + (((size_t)page * 2 + 1) * p.page_size + slot) * row_bytes);
  for (int i = threadIdx.x; i < 2 * chunks; i += blockDim.x) {
    if (i < chunks) {
      if constexpr (ROPE >= 0) {
        // this row's table entries of the chunk's pairs
        const size_t t = (size_t)r * (p.head_dim >> 1);
        f32x4 c, s;
        rope_entries<ROPE>(p.rope_cos + t, p.rope_sin + t, (uint32_t)i, p.head_dim, c, s);
        dk[i] = rope_chunk<ROPE>(sk[i], c, s);
      } else {
        dk[i] = sk[i];
      }
    } else {
      dv[i - chunks] = sv[i - chunks];
    }
  }
}

// Query rows [rows, H, D] -> rotated rows, one 16-byte chunk per thread.
template <int E>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;   // chunks < 2^31, checked by the host
  if (i >= (uint32_t)p.chunks) return;
  const uint32_t cpr = (uint32_t)p.row_elems / (E == 2 ? 4u : 8u);   // chunks per row
  const uint32_t row = i / cpr;
  const size_t t = (size_t)row * (uint32_t)(p.head_dim >> 1);
  f32x4 c, s;
  rope_entries<E>(p.cos + t, p.sin + t, i - row * cpr, p.head_dim, c, s);
  reinterpret_cast<u32x4*>(p.y)[i] = rope_chunk<E>(reinterpret_cast<const u32x4*>(p.x)[i], c, s);
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
template <int D>
struct Shape {
  static constexpr int CPR = D / 8;                      // 16-byte chunks per K/V row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int KSTEPS = D / 32;                  // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 16;                    // 16-row blocks of O^T
  static constexpr int HALF_BYTES = KT * ROW_BYTES;      // K (or V) part of a stage, [kv][d]
  static constexpr int STAGE_BYTES = 2 * HALF_BYTES;
  static constexpr int NSTAGE = 4;                       // LDS ring of stages
  static constexpr int DIST = 2;                         // stages loaded ahead (<= NSTAGE - 2)
  static constexpr int LOADS = STAGE_BYTES / 1024;       // 1 KiB direct-to-LDS loads per stage
  static constexpr int LOADS_PER_WAVE = LOADS / KVC_ATTN_WAVES;
};

// 16-byte chunk swizzle inside a K/V row of LDS (XORed into the chunk index).
// The LDS has 64 banks of 4 bytes; a 64-lane read is served 256 bytes at a
// time, by groups of lanes measured with the bank-conflict counters:
//  * ds_read_b128 (K operand): lanes {8a .. 8a+7} together with
//    {32+8a .. 32+8a+7}.  In such a group lane bits 0, 1, 2 and 5 vary, i.e.
//    K row bits 0, 1, 3 and chunk bit 1; row bit 4 and the other chunk bits
//    are fixed.
//  * ds_read_b64_tr_b16 (V^T operand): lanes 0-31, then 32-63.  In a group
//    lane bits 0-4 vary, i.e. V row bits 0, 1, 3, chunk bit 0 and the 8-byte
//    half; row bit 4 is fixed.
// A group must cover its 256-byte window one-to-one.  The bits of the window
// address are the row bits below the window (none for D=128, bit 0 for
// D=64, bits 0-1 for D=32) and the swizzled chunk, so the swizzle has to
// make the remaining varying bits a bijection: for D=64 swizzle bits {0, 2}
// over row bits {1, 3} (K) and {1, 2} over {1, 3} (V); for D=32 bit 0 and
// bit 1 over row bit 3; for D=128 bits {0, 2, 3} (K) and {1, 2, 3} (V) over
// row bits {0, 1, 3}.
template <int D>
__device__ __forceinline__ int swz(int row) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b3 = (row >> 3) & 1, b4 = (row >> 4) & 1;
  if constexpr (D == 32) return b3 | (b3 << 1);
  else if constexpr (D == 64) return b1 | ((b1 ^ b3) << 1) | ((b3 ^ b4) << 2);
  else return b3 | (b3 << 1) | (b0 << 2) | (b1 << 3);
}

template <int D, int E>
struct Ops {
  using S = Shape<D>;
  using T = El<E>;
  static constexpr int KS = S::KSTEPS;
  static constexpr int DB = S::DBLK;

  // S^T = K Q^T for the four 16-kv blocks of a stage
  static __device__ __forceinline__ void qk(const bf16x8 (&kop)[4][KS], const bf16x8 (&q)[KS], f32x4 (&s)[4]) {
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi) {
      s[kbi] = T::mfma(kop[kbi][0], q[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) s[kbi] = T::mfma(kop[kbi][ks], q[ks], s[kbi]);
    }
  }
  // the same for one 16-kv block
  static __device__ __forceinline__ void qk1(const bf16x8 (&k)[KS], const bf16x8 (&q)[KS], f32x4 (&s)[1]) {
    s[0] = T::mfma(k[0], q[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) s[0] = T::mfma(k[ks], q[ks], s[0]);
  }
  // O^T[D x 16 q] += V^T P^T over the stage's two 32-kv pairs
  static __device__ __forceinline__ void pv(const bf16x8 (&vop)[DB][2], const u32x4 (&pb)[2], f32x4 (&o)[DB]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        o[db] = T::mfma(vop[db][pp], __builtin_bit_cast(bf16x8, pb[pp]), o[db]);
  }
  // Column sums of P^T over the stage (both pairs): the same product with an
  // all-ones V^T, so every accumulator of a lane holds its query column's sum
  // of the rounded probabilities the P.V product uses.
  static __device__ __forceinline__ f32x4 colsum(const bf16x8& ones, const u32x4 (&pb)[2]) {
    const f32x4 c = T::mfma(ones, __builtin_bit_cast(bf16x8, pb[0]), f32x4{0.f, 0.f, 0.f, 0.f});
    return T::mfma(ones, __builtin_bit_cast(bf16x8, pb[1]), c);
  }
  // ... over one pair
  template <int PP>
  static __device__ __forceinline__ void pv1(const bf16x8 (&vop)[DB][2], const u32x4& pb, f32x4 (&o)[DB]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
      o[db] = T::mfma(vop[db][PP], __builtin_bit_cast(bf16x8, pb), o[db]);
  }
};

// p = 2^(s * scale - ref) packed in pairs in the element type (the P^T
// operand), and the lane's sum of the packed values (the same numbers the P.V
// product uses).  The packing rounds toward zero (for bf16 it keeps the upper
// half of the float32: one byte permute per pair): its relative error has the
// same spread as round-to-nearest (one ulp wide) and a mean of half an ulp,
// and numerator and denominator are sums over the same rounded weights, so
// that mean cancels in the normalisation.
template <int N, int E>
__device__ __forceinline__ float probs(const f32x4 (&s)[N], float sl, float nref, uint32_t (&pk)[2 * N]) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[i][2 * h], sl, nref)),
                                       __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][2 * h + 1], sl, nref)));
      pk[2 * i + h] = w;
      if (h == 0)
        a = El<E>::dot_ones(w, a);
      else
        b = El<E>::dot_ones(w, b);
    }
  return a + b;
}

// The same packing without the lane sum (the own tiles take their sums from
// the MFMA, colsum).
template <int N, int E>
__device__ __forceinline__ void probs_pack(const f32x4 (&s)[N], float sl, float nref, uint32_t (&pk)[2 * N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      pk[2 * i + h] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[i][2 * h], sl, nref)),
                                    __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][2 * h + 1], sl, nref)));
}

// Slots of score block j held by lane group g4 are boff[j] + 8 g4 + i (boff
// is the block's first slot); those at or past `valid` get score -inf
// (probability 0).  lim is valid - 8 g4, made opaque so that the compares
// stay inside the (rarely taken) branch of a partial stage.
template <int N>
__device__ __forceinline__ void mask_scores(f32x4 (&s)[N], const int (&boff)[N], int valid, int g4) {
  // rare branch: wait states first, clear of the MFMAs that wrote s
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  int lim = valid - 8 * g4;
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int j = 0; j < N; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (boff[j] + i >= lim) s[j][i] = -INFINITY;
}

// Exact path: column maximum of s * scale - ref over the stage (the four lane groups
// of a column hold its 64 slots), move ref up to it (while the tile has seen
// no valid slot yet, `fresh`: set it), scale the running sum and output by
// 2^-(shift), and recompute the probabilities.  Every column of a block has
// the same masked slots, so the maximum is -inf in all lanes or in none; a
// fresh tile whose slots were all masked stays fresh.  Taken rarely; a few
// wait states at both ends keep it clear of the MFMAs around it.
template <int N, int DB, int E>
__device__ __forceinline__ float renorm(const f32x4 (&s)[N], float sl, int& fresh, float& ref, float& nref,
                                        float& l, f32x4 (&o)[DB], uint32_t (&pk)[2 * N]) {
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  float m = s[0][0];
#pragma unroll
  for (int j = 0; j < N; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max2(m, s[j][i]);
  m = __builtin_fmaf(lane_swap_max(m), sl, nref);
  const bool first = fresh != 0;
  // uniform: kept in a scalar register
  fresh = __builtin_amdgcn_readfirstlane((int)(first && __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0));
  const float shift = first ? (m == -INFINITY ? 0.0f : m) : fmaxf(m, 0.0f);
  if (!first) {
    const float alpha = __builtin_amdgcn_exp2f(-shift);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
  }
  ref += shift;
  nref = -ref;
  const float lt = probs<N, E>(s, sl, nref, pk);
  asm volatile("s_nop 3" ::: "memory");
  return lt;
}

// Attention over one KV split for one head and one query group of up to
// 4 * 2 + 1 tiles of 16 queries.  Wave w owns tiles t_lo + w and t_lo + w + 4;
// the ninth tile (if the group has one) is shared: in every stage each wave
// takes one 16-kv block of it, and the four partial softmax states are merged
// at the end.  Every wave thus does the same work per stage (2.25 tiles), and
// the per-stage code is straight-line.
//
// Per stage s the wave runs three steps, one per tile (own 0, own 1, shared),
// each pairing one tile's probabilities (vector unit) with the MFMAs of its
// neighbours:
//   step 0: QK(s, own 1), PV(s-1, own 1), PV(s-1, shared) | probs(s, own 0)
//   step 1: QK(s, shared), PV(s, own 0)                   | probs(s, own 1)
//   step 2: QK(s+1, own 0)                                 | probs(s, shared)
// Each step is one straight-line block in which scheduling groups interleave
// the MFMAs with the vector work; the rare branches (partial-stage masking,
// the exact renormalisation) sit between the blocks.  After step 0, the V
// operands of stage s are read from LDS, stage s+1 is published (barrier)
// and its K operands are read, ahead of steps 1 and 2; the shared block's K
// of stage s+1 is read after step 1.  An MFMA result is read by the vector
// unit one step after its MFMA at the earliest.  After the last stage the same code
// reads a ring slot that holds no stage and computes a QK^T that is never
// used; every LDS address stays inside the ring.
template <int D, int E, bool SH>
__global__ __launch_bounds__(256, (D <= 64 ? 2 : 1)) void attn_kernel(AttnParams p) {
  using S = Shape<D>;
  using O = Ops<D, E>;
  constexpr int KS = S::KSTEPS;
  constexpr int DB = S::DBLK;
  constexpr int LPW = S::LOADS_PER_WAVE;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S::NSTAGE * S::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);   // same value, known uniform
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int shPP = wv >> 1, shTT = wv & 1;   // pair and half of this wave's shared block

  // Work-groups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of work items so one head's splits share an L2.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * p.items_per_xcd + (bid >> 3);
  if (item >= p.num_items) return;

  const kvc_dev_stream st = stream_of_item(p, item);

  int local = item - st.item0;
  const int grp = local % st.n_group;
  local /= st.n_group;
  const int split = local % st.n_split;
  const int h = local / st.n_split;

  const int nqt = (st.n_q + KVC_Q_TILE - 1) / KVC_Q_TILE;
  const int t_lo = grp * nqt / st.n_group;
  const int t_hi = (grp + 1) * nqt / st.n_group;
  const int ntile = t_hi - t_lo;
  const bool has_shared = SH && ntile == 4 * 2 + 1;
  const int n_own = has_shared ? 8 : ntile;
  const int u0 = split * st.n_units / st.n_split;
  const int u1 = (split + 1) * st.n_units / st.n_split;
  const int nstage = u1 - u0;
  const int H = p.num_heads;
  const uint32_t slot_bytes = (uint32_t)H * D * 2;

  // This split's work units: entry i describes stage i (the host planner
  // resolved pages, chunks and valid lengths).
  const int32_t* units = p.plan + st.unit0 + KVC_UNIT_INTS * u0;
  const uint64_t head_off = (uint64_t)h * D * 2;

  // ---- query operands: Q^T as the MFMA B operand
  const float sl = p.scale_log2;
  auto load_q = [&](int tile, bool ok, bf16x8 (&q)[KS]) {
    const int row = KVC_Q_TILE * tile + r16;
    ok = ok && row < st.n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)(st.q_row0 + (ok ? row : 0)) * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g4);
      if (!ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[ks][j] = (__bf16)0.0f;
      }
    }
  };
  bf16x8 q0[KS], q1[KS], q2[KS];
  load_q(t_lo + wave, wave < n_own, q0);
  load_q(t_lo + wave + 4, wave + 4 < n_own, q1);
  if constexpr (SH) load_q(t_hi - 1, has_shared, q2);

  // softmax state of tiles own 0, own 1, shared
  // ref of each tile and its negation; fresh: no valid slot seen yet (ref
  // not set)
  float ref0 = 0.f, ref1 = 0.f, ref2 = 0.f;
  float nref0 = 0.f, nref1 = 0.f, nref2 = 0.f;
  int fresh0 = 1, fresh1 = 1, fresh2 = 1;
  float l0 = 0.f, l1 = 0.f, l2 = 0.f;
  f32x4 o0[DB], o1[DB], o2[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o0[db] = o1[db] = o2[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- direct global -> LDS loads of one stage (K rows, then V rows) ----
  // Load instruction i of a stage fills 1 KiB of LDS, lane l writing bytes
  // [16 l, 16 l + 16); the lane fetches the logical chunk that the swizzle
  // places there, from the stage's uniform base address plus a per-lane
  // offset.  In a partial stage, rows past the valid count re-read the last
  // valid row (finite data; their scores are masked to -inf).
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  const uint64_t v_half = (uint64_t)p.page_size * slot_bytes;
  // row of the stage that lane fetches for load j, and its offset from the
  // stage base when every row is valid
  auto lrow = [&](int j) { return ((wave * LPW + j) % (S::LOADS / 2) * 1024 + lane * 16) / S::ROW_BYTES; };
  uint32_t vfull[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int off = (wave * LPW + j) % (S::LOADS / 2) * 1024 + lane * 16;
    const int row = off / S::ROW_BYTES;
    const int pch = (off % S::ROW_BYTES) >> 4;
    vfull[j] = (uint32_t)row * slot_bytes + (uint32_t)((pch ^ swz<D>(row)) << 4);
  }
  // LDS byte address of the ring (uniform)
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  auto issue = [&](int sidx, const i32x4& e) {
    const uint64_t koff = (uint64_t)(uint32_t)e.x * slot_bytes + head_off;
    const int valid = e.y;
    const uint32_t slot = ring_lds + (uint32_t)(sidx % S::NSTAGE) * S::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int inst = wv * LPW + j;
      const int kv = inst >= S::LOADS / 2 ? 1 : 0;
      const int blk = inst - kv * (S::LOADS / 2);
      uint32_t vofs = vfull[j];
      if (valid < KT) {
        const int row = lrow(j);
        vofs -= (uint32_t)(row - min(row, valid - 1)) * slot_bytes;
      }
      load_lds16(pool + koff + (kv ? v_half : 0), vofs, slot + (uint32_t)(kv * S::HALF_BYTES + blk * 1024));
    }
  };

  // ---- operand reads from a published stage ----
  // K operand rows: block kbi (= 2*pair + half) row r16 holds kv
  // 32*pair + 8*(r16/4) + 4*half + r16%4, so that after the MFMA lane group
  // g4 holds kv 32*pair + 8*g4 + 4*half + [0, 4) of each query column.
  // The shared tile's block of wave w is the 16 slots 32*(w/2) + 4*(w%2) +
  // {8 g + i}.  A wave whose block lies in the second 32-slot pair swaps the
  // two pairs in all its operands: operand pair p holds slots of pair
  // p ^ shPP, in the K rows (hence in the scores and the P^T operand) and in
  // V^T alike, so every product is unchanged and the shared block's V^T is
  // always operand pair 0.
  //
  // The row of a K operand read is 32*pair + 4*(kbi%2) + kr (kr per lane,
  // bits 0, 1, 3, 4), that of a V read 32*pair + 4*r + vr (vr per lane, bits
  // 0, 1, 3, 4): the added bits 2 and 5 leave the swizzle unchanged, so every
  // read is a per-lane offset plus a compile-time constant.
  const int kr = 8 * (r16 >> 2) + (r16 & 3);
  const int vr = 8 * g4 + (r16 >> 2);
  uint32_t kofs[2][KS], kshofs[KS], vofs_l[2][DB];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int pair_rows = 32 * (pp ^ shPP) * S::ROW_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kofs[pp][ks] = (uint32_t)(pair_rows + kr * S::ROW_BYTES + (((4 * ks + g4) ^ swz<D>(kr)) << 4));
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vofs_l[pp][db] = (uint32_t)(pair_rows + S::HALF_BYTES + vr * S::ROW_BYTES +
                                  (((2 * db + ((r16 & 3) >> 1)) ^ swz<D>(vr)) << 4) + ((r16 & 1) << 3));
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kshofs[ks] = kofs[0][ks] + 4 * shTT * S::ROW_BYTES;
  auto read_k = [&](int sidx, bf16x8 (&kop)[4][KS]) {
    const uint8_t* kb = ring + (sidx % S::NSTAGE) * S::STAGE_BYTES;
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[kbi][ks] = *reinterpret_cast<const bf16x8*>(kb + kofs[kbi >> 1][ks] + 4 * (kbi & 1) * S::ROW_BYTES);
  };
  auto read_ksh = [&](int sidx, bf16x8 (&k)[KS]) {
    const uint8_t* kb = ring + (sidx % S::NSTAGE) * S::STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k[ks] = *reinterpret_cast<const bf16x8*>(kb + kshofs[ks]);
  };
  // V^T operands by transposing reads of row-major V: lane (g4, r16) gets
  // V[32*(pair ^ shPP) + 8*g4 + j][16*db + r16], j = 0..7.
  auto read_v = [&](int sidx, bf16x8 (&vop)[DB][2]) {
    const uint8_t* vb = ring + (sidx % S::NSTAGE) * S::STAGE_BYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        i16x4 half[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) half[r] = ds_read_tr16(vb + vofs_l[pp][db] + 4 * r * S::ROW_BYTES);
        const i16x4 a = half[0], b = half[1];
        vop[db][pp] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){a[0], a[1], a[2], a[3],
                                                                                             b[0], b[1], b[2], b[3]});
      }
  };

  // first slot of each score block (after the pair swap) for masking
  const int kb_own[4] = {32 * shPP, 32 * shPP + 4, 32 * (1 - shPP), 32 * (1 - shPP) + 4};
  const int kb_sh[1] = {32 * shPP + 4 * shTT};

  bf16x8 kop[4][KS], ksh[KS], vop[DB][2];
  // Own tiles' stage sums: by MFMA (colsum, an all-ones V^T operand)
  bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{El<E>::ONE2, El<E>::ONE2, El<E>::ONE2, El<E>::ONE2});
  // held in vector registers for the whole loop, not rebuilt before each use
  asm volatile("" : "+v"(ones));
  f32x4 sc0[4], sc1[4], sc2[1];
  uint32_t pk0[8], pk1[8], pk2[2];
  u32x4 pbsh = u32x4{0u, 0u, 0u, 0u};

  // ---- prologue: fill the ring, publish stage 0, issue its first QK ----
  // Unit entries are read three stages ahead; vq holds the valid counts of
  // stages s, s+1, s+2.
  i32x4 e0 = unit_load(units), e1 = unit_load(units + KVC_UNIT_INTS * min(1, nstage - 1)),
        e2 = unit_load(units + KVC_UNIT_INTS * min(2, nstage - 1));
  unit_wait(e0);
  unit_wait(e1);
  unit_wait(e2);
  issue(0, e0);
  if (nstage > 1) issue(1, e1);
  if (nstage > 2) issue(2, e2);
  int vq0 = e0.y, vq1 = e1.y, vq2 = e2.y;
  if (nstage >= 3)
    wait_vmcnt<2 * LPW>();
  else if (nstage == 2)
    wait_vmcnt<LPW>();
  else
    wait_vmcnt<0>();
  block_barrier();
  read_k(0, kop);
  if constexpr (SH) read_ksh(0, ksh);
  O::qk(kop, q0, sc0);

  // Stage 0's step 0 multiplies the zero P^T operands of "stage -1" with
  // zero V^T operands: exact zeros, so the loop needs no first-stage branch.
#pragma unroll
  for (int db = 0; db < DB; ++db) vop[db][0] = vop[db][1] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int i = 0; i < 8; ++i) pk1[i] = 0u;

  for (int s = 0; s < nstage; ++s) {
    const int valid = vq0;
    const bool partial = valid < KT;
    i32x4 en = unit_load(units + KVC_UNIT_INTS * min(s + 3, nstage - 1));

    // ---- step 0: MFMAs of own tile 1 and the shared tile | probabilities of own tile 0 ----
    if (partial) mask_scores<4>(sc0, kb_own, valid, g4);
    if constexpr (SH) O::template pv1<0>(vop, pbsh, o2);
    {
      u32x4 pb[2] = {u32x4{pk1[0], pk1[1], pk1[2], pk1[3]}, u32x4{pk1[4], pk1[5], pk1[6], pk1[7]}};
      O::pv(vop, pb, o1);
    }
    O::qk(kop, q1, sc1);
    probs_pack<4, E>(sc0, sl, nref0, pk0);
    const f32x4 cs0 =
        O::colsum(ones, {u32x4{pk0[0], pk0[1], pk0[2], pk0[3]}, u32x4{pk0[4], pk0[5], pk0[6], pk0[7]}});
    // one MFMA, then two vector instructions, while both last
#pragma unroll
    for (int i = 0; i < (SH ? 20 : 16); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    // The V operands of stage s (published one stage ago) are read once the
    // products above have consumed those of stage s-1; then stage s+1 is
    // published and its K operands read.  Every read of stage s-1 has
    // completed (the products above consumed them) before the barrier lets
    // the ring slot of stage s-1 be refilled.
    read_v(s, vop);
    if (s + 2 < nstage)
      wait_vmcnt<LPW>();
    else
      wait_vmcnt<0>();
    block_barrier();
    unit_wait(en);
    if (s + 3 < nstage) issue(s + 3, en);
    vq0 = vq1;
    vq1 = vq2;
    vq2 = en.y;
    read_k(s + 1, kop);

    // ---- step 1: QK of the shared tile, P.V of own tile 0 | probabilities of own tile 1 ----
    if (partial) mask_scores<4>(sc1, kb_own, valid, g4);
    if constexpr (SH) O::qk1(ksh, q2, sc2);
    // own tile 0: check its stage sum before its P.V
    float lt = cs0[0];
    if (fresh0 || __builtin_amdgcn_ballot_w64(sum_exceeds(lt, LAZY_COL_LIMIT)))
      lt = lane_swap_sum(renorm<4, DB, E>(sc0, sl, fresh0, ref0, nref0, l0, o0, pk0));
    l0 += lt;
    {
      u32x4 pb[2] = {u32x4{pk0[0], pk0[1], pk0[2], pk0[3]}, u32x4{pk0[4], pk0[5], pk0[6], pk0[7]}};
      O::pv(vop, pb, o0);
    }
    probs_pack<4, E>(sc1, sl, nref1, pk1);
    const f32x4 cs1 =
        O::colsum(ones, {u32x4{pk1[0], pk1[1], pk1[2], pk1[3]}, u32x4{pk1[4], pk1[5], pk1[6], pk1[7]}});
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    if constexpr (SH) read_ksh(s + 1, ksh);

    // ---- step 2: QK of own tile 0 for stage s+1 | probabilities of the shared tile ----
    if constexpr (SH) {
      if (partial) mask_scores<1>(sc2, kb_sh, valid, g4);
    }
    O::qk(kop, q0, sc0);
    float lt2 = 0.f;
    if constexpr (SH) {
      lt2 = probs<1, E>(sc2, sl, nref2, pk2);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      // keep the shared tile's probabilities here, beside the MFMAs above,
      // rather than sunk past the branch below
      asm volatile("" : "+v"(lt2));
    }
    // own tile 1: check its stage sum (its P.V follows in the next step 0)
    lt = cs1[0];
    if (fresh1 || __builtin_amdgcn_ballot_w64(sum_exceeds(lt, LAZY_COL_LIMIT)))
      lt = lane_swap_sum(renorm<4, DB, E>(sc1, sl, fresh1, ref1, nref1, l1, o1, pk1));
    l1 += lt;
    if constexpr (SH) {
      if (fresh2 || __builtin_amdgcn_ballot_w64(sum_exceeds(lt2, LAZY_SUM_LIMIT)))
        lt2 = renorm<1, DB, E>(sc2, sl, fresh2, ref2, nref2, l2, o2, pk2);
      l2 += lt2;
      // P^T of the shared block: its 4 slots sit at positions 4*half..4*half+3
      // of the pair's operand; the other half is zero
      pbsh = shTT ? u32x4{0u, 0u, pk2[0], pk2[1]} : u32x4{pk2[0], pk2[1], 0u, 0u};
    }
  }
  if constexpr (SH) O::template pv1<0>(vop, pbsh, o2);
  {
    u32x4 pb[2] = {u32x4{pk1[0], pk1[1], pk1[2], pk1[3]}, u32x4{pk1[4], pk1[5], pk1[6], pk1[7]}};
    O::pv(vop, pb, o1);
  }

  // The epilogue reads the accumulators the last MFMAs wrote; give those
  // MFMAs their result latency regardless of how the loop exit is laid out.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- epilogue ----
  auto store = [&](int tile, float ref, float l, const f32x4 (&o)[DB]) {
    const float inv = 1.0f / l;
    const int row = KVC_Q_TILE * tile + r16;
    if (st.n_split > 1) {
      // normalised partial output, rounded to bf16 (a convex combination of
      // V rows, so within V's range), and its log-sum-exp in float32; rows
      // past the stream's queries are stored too (finite; never merged).
      // The layout is that of the 32x32 kernel's accumulators (per 32-row
      // tile): this 16-row tile is half `tile & 1` of 32-row tile tile / 2,
      // and lane (r16, g4)'s four values of d block db are d = 16 db + 4 g4
      // .. + 3, i.e. 32-lane row 16 (tile & 1) + r16 of slice (d / 32,
      // (d % 32) / 8), lane half (d / 4) & 1.
      const size_t pt = ((size_t)split * H + h) * p.tiles_cap + st.q_tile0 + (tile >> 1);
      const int r32 = 16 * (tile & 1) + r16;
      uint16_t* po = static_cast<uint16_t*>(p.part_o) + pt * (size_t)(D / 32 * 4 * 256);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + 4 * g4;
        *reinterpret_cast<u32x2*>(po + ((d >> 5) * 4 + ((d & 31) >> 3)) * 256 + (32 * ((d >> 2) & 1) + r32) * 4) =
            El<E>::cvt4(o[db] * inv);
      }
      if (g4 == 0) p.part_lse[pt * KVC_Q_TILE32 + r32] = ref + __log2f(l);
      return;
    }
    if (row >= st.n_q) return;
    const int grow = st.q_row0 + row;
    {
      uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)grow * H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g4) = El<E>::cvt4(o[db] * inv);
    }
  };
  // l0 and l1 are whole column sums (the column-sum MFMAs); l2 is the lane
  // group's share, summed in the shared tile's merge below
  if (wave < n_own) store(t_lo + wave, ref0, l0, o0);
  if (wave + 4 < n_own) store(t_lo + wave + 4, ref1, l1, o1);

  if (has_shared) {
    // merge the four waves' partial states of the shared tile (one split
    // merge: weights 2^(ref_w - max ref))
    constexpr int NV = DB * 4 + 2;
    float* xs = reinterpret_cast<float*>(ring);
    const float lt2 = lane_swap_sum(l2);
    __syncthreads();   // every wave is done with the ring
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[(wave * 64 + lane) * NV + 4 * db + i] = o2[db][i];
    // a wave whose block of the shared tile held no valid slot has l = 0
    xs[(wave * 64 + lane) * NV + DB * 4] = lt2 > 0.0f ? ref2 : -INFINITY;
    xs[(wave * 64 + lane) * NV + DB * 4 + 1] = lt2;
    __syncthreads();
    if (wave == 0) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < KVC_ATTN_WAVES; ++w) M = fmaxf(M, xs[(w * 64 + lane) * NV + DB * 4]);
      float lsum = 0.f;
      f32x4 o[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < KVC_ATTN_WAVES; ++w) {
        const float* x = xs + (w * 64 + lane) * NV;
        const float wt = __builtin_amdgcn_exp2f(x[DB * 4] - M);
        lsum += wt * x[DB * 4 + 1];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[db][i] += wt * x[4 * db + i];
      }
      store(t_hi - 1, M, lsum, o);
    }
  }
}

// ---------------------------------------------------------------------------
// attention on float32 pools
// ---------------------------------------------------------------------------
// The full-precision variant ([p3] FAQ on fp32 precision; [p4] §Memory
// Management and Debugging): K, V, Q and O in float32, products and sums in
// float32 on v_mfma_f32_16x16x4_f32, the online softmax in float32 (exact:
// the running maximum moves at every stage) and the probabilities not
// rounded.  Work item = (stream, head, 16-query tile), one work-group of
// F32_WAVES waves: wave w takes units w, w + F32_WAVES, ... of the stream, and
// the waves' softmax states are merged through LDS at the end (no split
// across work-groups, hence no merge launch).
//
// Scores are transposed, S^T = K Q^T, per 16-slot block b of a unit: kv on
// the rows, queries on the columns.  The contraction index d is assigned to
// (k-step ks, lane group g = l / 16) as d = (D / 4) g + ks, so each lane reads
// a contiguous quarter of a K row and of its query row.  Lane l then holds
// the scores of query l % 16 with slots 16 b + 4 g + j (j = 0..3), and
// O^T = V^T P^T takes k-step (b, j) with lane group g contributing slot
// 16 b + 4 g + j: the B operand is the lane's own probability j.
constexpr int F32_WAVES = 8;

template <int D>
__global__ __launch_bounds__(64 * F32_WAVES) void attn_f32_kernel(AttnParams p) {
  constexpr int KQ = D / 4;    // contraction steps per block = floats per lane quarter
  constexpr int DB = D / 16;   // 16-row blocks of O^T
  constexpr int NV = 4 * DB + 2;   // floats per lane of a wave's state: O^T, max, sum
  __shared__ float xs[F32_WAVES * 64 * NV];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int item = blockIdx.x;
  const kvc_dev_stream st = stream_of_item(p, item);
  const int local = item - st.item0;
  const int tile = local % st.n_group;   // groups of one 16-row tile; one split
  const int hd = local / st.n_group;
  const int H = p.num_heads;
  const int n = lane & 15, g = lane >> 4;
  const size_t slot_elems = (size_t)H * D;
  const float sl = p.scale_log2;

  float qv[KQ];
  {
    const int row = min(16 * tile + n, st.n_q - 1);
    const f32x4* qp = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) +
                                                     ((size_t)(st.q_row0 + row) * H + hd) * D + KQ * g);
#pragma unroll
    for (int i = 0; i < KQ / 4; ++i) {
      const f32x4 x = qp[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[4 * i + j] = x[j];
    }
  }
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;   // running maximum of s * scale (log2 units) and sum

  const float* pool = static_cast<const float*>(p.pool);
  const int32_t* units = p.plan + st.unit0;
  for (int u = wv; u < st.n_units; u += F32_WAVES) {
    const uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane(units[KVC_UNIT_INTS * u]);
    const int valid = __builtin_amdgcn_readfirstlane(units[KVC_UNIT_INTS * u + 1]);
    const float* kb = pool + (size_t)slot * slot_elems + (size_t)hd * D;   // K of the unit's first slot
    const float* vb = kb + (size_t)p.page_size * slot_elems;              // its V
    f32x4 sc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // rows past the valid count re-read the last valid one (masked below)
      const f32x4* kp = reinterpret_cast<const f32x4*>(kb + (size_t)min(16 * b + n, valid - 1) * slot_elems + KQ * g);
      float kq[KQ];
#pragma unroll
      for (int i = 0; i < KQ / 4; ++i) {
        const f32x4 x = kp[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) kq[4 * i + j] = x[j];
      }
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) sc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(kq[ks], qv[ks], sc[b], 0, 0, 0);
    }
    // scores in log2 units; slots at or past `valid` masked
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = 16 * b + 4 * g + j < valid ? sc[b][j] * sl : -INFINITY;
        sc[b][j] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    // nothing valid seen yet: keep everything at zero
    const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[b][j] - mn);
        sc[b][j] = e;
        rs += e;
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* vr = vb + (size_t)min(16 * b + 4 * g + j, valid - 1) * slot_elems;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[16 * db + n], sc[b][j], o[db], 0, 0, 0);
      }
  }
  // merge the waves' states (weights 2^(m_w - max m); a wave that saw no
  // valid slot has m = -inf and weighs nothing)
  {
    float* x = xs + (wv * 64 + lane) * NV;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * db + r] = o[db][r];
    x[4 * DB] = m;
    x[4 * DB + 1] = l;
  }
  __syncthreads();
  if (wv != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < F32_WAVES; ++w) M = fmaxf(M, xs[(w * 64 + lane) * NV + 4 * DB]);
  float lsum = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < F32_WAVES; ++w) {
    const float* x = xs + (w * 64 + lane) * NV;
    const float wt = x[4 * DB] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[4 * DB] - M);
    lsum += wt * x[4 * DB + 1];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[db][r] += wt * x[4 * db + r];
  }
  // lane l holds O^T[16 db + 4 g + r][query n] in element r of block db
  const int row = 16 * tile + n;
  if (row < st.n_q) {
    const float inv = 1.0f / lsum;
    float* orow = static_cast<float*>(p.o) + ((size_t)(st.q_row0 + row) * H + hd) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(orow + 16 * db + 4 * g) = o[db] * inv;
  }
}

// ---------------------------------------------------------------------------
// merge of KV splits
// ---------------------------------------------------------------------------
// One work-group per (32-row query tile, head) of a split stream, on the XCD
// whose L2 holds most of its partials (the plan's merge order lists the
// pairs of each XCD; work-group b runs on XCD b % 8).  The partials are laid
// out per tile as D / 32 x 4 slices of 64 lanes x 4 values (the 32x32
// accumulator order); wave w takes slice w, each lane the 4 values it holds
// in every split: row n = lane % 32, d = 32 (w / 4) + 8 (w % 4) + 4 (lane / 32)
// .. + 3.  The pair's merge-order entry gives its stream's split count and
// output rows.  The partials and log-sum-exps of up to CH splits are loaded
// together, then folded in split order with weights 2^(lse_c - running max):
// one memory round trip per chunk, and every sum in a fixed order.  Splits
// past the tile's own count (other streams may have more) are never loaded.
// Fused append: the step's input rows into the pool, 16 bytes per thread
// and copy, COPY_PER copies per thread with their loads issued together.
// Copy q of the launch is chunk q % cpr of the K (q / cpr even) or V half of
// input row q / (2 cpr).
constexpr int COPY_PER = KVC_COPY_PER;
__device__ __forceinline__ void copy_own_rows(const MergeParams& p, int wg, int nthreads) {
  const uint32_t cpr = (uint32_t)p.row_bytes >> 4;
  const uint32_t total = (uint32_t)p.copy_rows * 2u * cpr;
  const uint32_t q0 = (uint32_t)wg * (uint32_t)nthreads * COPY_PER + threadIdx.x;
  u32x4 x[COPY_PER];
  u32x4* dst[COPY_PER];
#pragma unroll
  for (int k = 0; k < COPY_PER; ++k) {
    const uint32_t q = q0 + (uint32_t)(k * nthreads);
    dst[k] = nullptr;
    if (q < total) {
      const uint32_t row = q / (2u * cpr);
      const uint32_t rem = q - row * 2u * cpr;
      const bool vh = rem >= cpr;
      const uint32_t ch = vh ? rem - cpr : rem;
      int si = 0;
#pragma unroll
      for (int i = 1; i < KVC_ARG_STREAMS; ++i)
        if (i < p.num_streams && (int)row >= p.row0[i]) si = i;
      const uint8_t* src = static_cast<const uint8_t*>(vh ? p.vin[si] : p.kin[si]) +
                           (size_t)(row - (uint32_t)p.row0[si]) * p.row_bytes + 16u * ch;
      const uint32_t kslot = (uint32_t)p.plan[p.copy_table + row];
      dst[k] = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.pool) +
                                        ((size_t)kslot + (vh ? (size_t)p.page_size : 0)) * p.row_bytes + 16u * ch);
      x[k] = *reinterpret_cast<const u32x4*>(src);
    }
  }
#pragma unroll
  for (int k = 0; k < COPY_PER; ++k)
    if (dst[k]) *dst[k] = x[k];
}

template <int D, int E, int CH>
// plan, merge_table and merge_slots repeat fields of p as leading scalar
// arguments, which the dispatch preloads into scalar registers: the merge
// order's entry is then read without waiting for the argument segment.
__global__ __launch_bounds__(64 * (D / 32) * 4) void merge_kernel(const int32_t* __restrict__ plan,
                                                                   int32_t merge_table, int32_t merge_slots,
                                                                   MergeParams p) {
  constexpr int SLICES = D / 32 * 4;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int H = p.num_heads;
  if ((int)blockIdx.x >= KVC_NUM_XCD * merge_slots) {   // uniform over the work-group
    copy_own_rows(p, (int)blockIdx.x - KVC_NUM_XCD * merge_slots, 64 * (D / 32) * 4);
    return;
  }
  const int slot = blockIdx.x >> 3;
  // {tile * H + head, splits, first output row, valid rows}
  const i32x4 te = *reinterpret_cast<const i32x4*>(
      plan + merge_table + KVC_MERGE_INTS * ((blockIdx.x & (KVC_NUM_XCD - 1)) * merge_slots + slot));
  const int pair = te.x;
  if (pair < 0) return;
  const int gt = pair / H;                // global 32-row tile
  const int h = pair - gt * H;
  const int nsp = te.y;
  const int n = lane & 31, hh = lane >> 5;
  const size_t tstride = (size_t)H * p.tiles_cap;   // between splits, in tiles
  const size_t t0 = (size_t)h * p.tiles_cap + gt;
  const uint16_t* po = static_cast<const uint16_t*>(p.part_o) + (t0 * SLICES + w) * 256 + lane * 4;
  const float* pl = p.part_lse + t0 * KVC_Q_TILE32 + n;
  float m = -INFINITY, wsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nsp; c0 += CH) {
    float lse[CH];
    u32x2 x[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (c0 + j < nsp) {
        const size_t c = (size_t)(c0 + j) * tstride;
        lse[j] = pl[c * KVC_Q_TILE32];
        x[j] = *reinterpret_cast<const u32x2*>(po + c * SLICES * 256);
      }
    float mc = m;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (c0 + j < nsp) mc = fmaxf(mc, lse[j]);
    if (mc == -INFINITY) continue;        // nothing of weight yet
    const float sc = __builtin_amdgcn_exp2f(m - mc);   // 0 while m is -inf
    acc *= sc;
    wsum *= sc;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (c0 + j < nsp) {
        const float wt = __builtin_amdgcn_exp2f(lse[j] - mc);
        acc += wt * El<E>::widen4(x[j]);
        wsum += wt;
      }
    m = mc;
  }
  if (n < te.w) {
    const int d = 32 * (w >> 2) + 8 * (w & 3) + 4 * hh;
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ((size_t)(te.z + n) * H + h) * D + d) =
        El<E>::cvt4(acc * (1.0f / wsum));
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// static scratch of kvc_run_no_alloc
// ---------------------------------------------------------------------------
// Split partial outputs of kvc_run_no_alloc.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address (one per device,
// each device holding its own copy) comes from hipGetSymbolAddress, and only
// that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[KVC_NO_ALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices] = {};
}  // namespace

int no_alloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  *bytes = KVC_NO_ALLOC_SCRATCH_BYTES;
  return 0;
}

int launch_append(const AppendParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  if (!p.rope_cos)
    hipLaunchKernelGGL(append_kernel<-1>, dim3(p.T), dim3(256), 0, hs, p);
  else if (p.dtype == 0)
    hipLaunchKernelGGL(append_kernel<0>, dim3(p.T), dim3(256), 0, hs, p);
  else if (p.dtype == 1)
    hipLaunchKernelGGL(append_kernel<1>, dim3(p.T), dim3(256), 0, hs, p);
  else if (p.dtype == 2)
    hipLaunchKernelGGL(append_kernel<2>, dim3(p.T), dim3(256), 0, hs, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_rope(const RopeParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  if (p.chunks == 0) return 0;
  const dim3 grid((unsigned)((p.chunks + 255) / 256));
  if (p.dtype == 0)
    hipLaunchKernelGGL(rope_kernel<0>, grid, dim3(256), 0, hs, p);
  else if (p.dtype == 1)
    hipLaunchKernelGGL(rope_kernel<1>, grid, dim3(256), 0, hs, p);
  else if (p.dtype == 2)
    hipLaunchKernelGGL(rope_kernel<2>, grid, dim3(256), 0, hs, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// Instantiations by (D, element type).  The 16x16 attention kernel serves
// head_dim 128, and 64 where the plan picks it (the multi-frame scale step);
// otherwise 32 and 64 go to the 32x32 kernel (kvc_attn.hip).
template <int E, bool SH>
static int launch_attention_es(const AttnParams& p, int32_t grid, hipStream_t hs) {
  if (p.head_dim == 128)
    hipLaunchKernelGGL((attn_kernel<128, E, SH>), dim3(grid), dim3(256), 0, hs, p);
  else if constexpr (!SH) {
    // head_dim 64 in 16-row tiles (two work-groups per CU) for plans with few
    // query tiles; the shared-tile form does not fit the registers there
    if (p.head_dim != 64) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<64, E, false>), dim3(grid), dim3(256), 0, hs, p);
  } else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

template <int E>
static int launch_attention_e(const AttnParams& p, int32_t grid, hipStream_t hs) {
  return p.shared_tile ? launch_attention_es<E, true>(p, grid, hs) : launch_attention_es<E, false>(p, grid, hs);
}

int launch_attention(const AttnParams& p, int32_t grid, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  if (p.dtype == 0) return launch_attention_e<0>(p, grid, hs);
  if (p.dtype == 1) return launch_attention_e<1>(p, grid, hs);
  return (int)hipErrorInvalidValue;
}

int launch_attention_f32(const AttnParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  const dim3 grid((unsigned)p.num_items), block(64 * F32_WAVES);
  if (p.num_items == 0) return 0;
  switch (p.head_dim) {
    case 32:
      hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, hs, p);
      break;
    case 64:
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, hs, p);
      break;
    case 128:
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, hs, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int E, int CH>
static int launch_merge_ec(const MergeParams& p, int grid, hipStream_t hs) {
  switch (p.head_dim) {
    case 32:
      hipLaunchKernelGGL((merge_kernel<32, E, CH>), dim3(grid), dim3(64 * 4), 0, hs, p.plan, p.merge_table,
                         p.merge_slots, p);
      break;
    case 64:
      hipLaunchKernelGGL((merge_kernel<64, E, CH>), dim3(grid), dim3(64 * 8), 0, hs, p.plan, p.merge_table,
                         p.merge_slots, p);
      break;
    case 128:
      hipLaunchKernelGGL((merge_kernel<128, E, CH>), dim3(grid), dim3(64 * 16), 0, hs, p.plan, p.merge_table,
                         p.merge_slots, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Chunk: the smallest of 4, 8, 16 that covers the largest split count, else
// 16 (two or more round trips).
template <int E>
static int launch_merge_e(const MergeParams& p, int grid, hipStream_t hs) {
  if (p.max_split <= 4) return launch_merge_ec<E, 4>(p, grid, hs);
  if (p.max_split <= 8) return launch_merge_ec<E, 8>(p, grid, hs);
  return launch_merge_ec<E, 16>(p, grid, hs);
}

int launch_merge(const MergeParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  // one work-group per merged (query tile, head), then the copy work-groups
  const int grid = KVC_NUM_XCD * p.merge_slots + p.copy_wgs;
  if (grid == 0) return 0;
  if (p.dtype == 0) return launch_merge_e<0>(p, grid, hs);
  if (p.dtype == 1) return launch_merge_e<1>(p, grid, hs);
  return (int)hipErrorInvalidValue;
}

}  // namespace kvc
