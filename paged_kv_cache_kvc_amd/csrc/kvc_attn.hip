// Paged prefill attention for head_dim 32 and 64 on gfx950 (MI355X), with
// 32x32x16 MFMAs.
//
// What it computes: for every planned stream, head and query row of the step,
// o = softmax(q K^T / sqrt(D)) V over the stream's valid visible tokens,
// unmasked, K and V gathered through the page table ([p2] "How LingBot-Map
// Uses FlashInfer KV Cache for Streaming 3D Reconstruction" §Attention Kernel
// Execution; [p1] "How FlashInfer KV Cache Attention Accelerates Streaming 3D
// Reconstruction Over SDPA" §Efficient Attention Masking and Padding: lengths
// delimit the valid tokens).  With split-KV each split writes its normalised
// partial output and log-sum-exp; the merge kernel combines them.
//
// Work item = (stream, head, KV split, query group).  A work-group of 4 waves
// (one per SIMD) streams its split's K/V through a ring of LDS stages of 64
// slots of one page, loaded by direct global-to-LDS loads.  A query group is
// up to 8 tiles of 32 queries: wave w owns tiles w (A) and w + 4 (B).  When
// the stream's rows leave a remainder of at most 16, those rows form a tail
// tile of 16 queries shared by the four waves: in every stage wave w takes
// its slots 16w .. 16w + 15 (16x16 MFMAs), and the four partial softmax
// states are merged at the end.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: kv
// slots on the rows, queries on the columns, so a lane's accumulators belong
// to one query (lane n and n + 32 hold its 64 slots, 32 each).  K rows are
// read in an order (bits 2 and 3 of the row swapped) that makes each lane's
// 8 consecutive accumulators the 8 consecutive slots the P.V product wants
// from that lane, so the probabilities pack straight into the P^T operand of
// O^T = V^T P^T.  V^T comes from row-major V by transposing LDS reads.
//
// Each stage runs two steps; each pairs one tile's softmax (vector unit) with
// the other tile's MFMAs:
//   step X: QK(B, s), PV(B, s-1), tail QK(s), tail PV(s-1) | softmax(A, s)
//   step Y: QK(A, s+1), PV(A, s)                           | softmax(B, s), tail softmax(s)
// Between them one barrier publishes stage s+1 and frees the ring slot of
// stage s-1; V(s) and K(s+1) are then read from LDS into registers, where they
// serve both tiles.  Probability row sums come from MFMAs against a 0/1 mask
// operand (below), a step before the lazy check that reads them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_device.h"
#include "kvc_kernels.h"

namespace kvc {

namespace {

using namespace dev;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <int E>
struct M32;

template <>
struct M32<0> {
  static __device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <>
struct M32<1> {
  static __device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                 0, 0);
  }
};

template <int D>
struct Shape32 {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int KS = D / 16;                    // k-steps of S^T = K Q^T (32x32x16)
  static constexpr int DB = D / 32;                    // 32-row blocks of O^T
  static constexpr int TKS = D / 32;                   // tail: k-steps of 16x16x32
  static constexpr int TDB = D / 16;                   // tail: 16-row blocks of O^T
  static constexpr int HALF = KVC_KV_TILE * ROW_BYTES; // K (or V) part of a stage
  static constexpr int STAGE = 2 * HALF;
  static constexpr int NSTAGE = 128 * 1024 / STAGE;    // ring of 128 KiB: 8 stages (D = 64), 16 (D = 32);
                                                       // NSTAGE - 2 stay in flight
  static constexpr int LOADS = STAGE / 1024;           // 1 KiB direct-to-LDS loads per stage
  static constexpr int LPW = LOADS / KVC_ATTN32_WAVES;
  static constexpr int QT = 32 * ROW_BYTES / 1024;     // loads per 32-row query tile
  static constexpr int TQ = 16 * ROW_BYTES / 1024;     // loads per 16-row tail
};

// 16-byte chunk swizzle inside a K/V row of LDS, XORed into the chunk index.
// A 64-lane LDS read is served 256 bytes at a time: a ds_read_b128 by lanes
// {8a .. 8a+7} with {32+8a .. 32+8a+7}, a ds_read_b64_tr_b16 by lanes 0-31,
// then 32-63.  In a K read group the rows vary in bits 0, 1, 3 (bits 2 and 3
// of the lane's row are swapped) and the chunk in bit 0; in a V read group
// the rows vary in bits 0, 1 and the chunk in bits 0, 1 plus the 8-byte
// half.  Row bit 0 picks the 128-byte half of the window (D = 64) or rows
// bits 0-1 its 64-byte quarter (D = 32); the swizzle maps the remaining
// varying bits one-to-one onto the chunk bits: D = 64: chunk ^= (row1 << 2)
// | (row3 << 1) | row2; D = 32: chunk ^= (row3 << 1) | row2 (row2 spreads the
// tail's K reads).
template <int D>
__device__ __forceinline__ int swz32(int row) {
  const int b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
  if constexpr (D == 64) return (b1 << 2) | (b3 << 1) | b2;
  else return (b3 << 1) | b2;
}

// K row read by lane row m of a 32-slot block: m with bits 2 and 3 swapped.
// Accumulator element e = 4i + j of lane (n, h) then holds slot
// 16 (i >> 1) + 8h + 4 (i & 1) + j of the block: elements 8u .. 8u + 7 are
// slots 16u + 8h .. 16u + 8h + 7, one lane's share of P.V k-step u.
__device__ __forceinline__ int kperm(int m) { return (m & 0x13) | ((m >> 1) & 0x4) | ((m << 1) & 0x8); }

// Row sums of P^T over one 16-slot k-step by a 16x16x32 MFMA: its B operand
// is the P^T register as is, which that MFMA reads as lanes {n16, n16 + 16,
// n16 + 32, n16 + 48} x 8 values: queries n16 and n16 + 16, each from both
// halves.  The A operand row m selects the lanes of query n16 + 16 ((m / 4)
// odd) or n16 ((m / 4) even), so result row 4g + j (held by lane 16g + n16)
// is the sum for query n16 + 16 (g & 1): the lane's own query.  Lane l's A
// operand is 8 ones when bit 2 of l equals bit 4, else zeros.
template <int E>
__device__ __forceinline__ bf16x8 rowsum_mask(int lane) {
  const uint32_t w = (((lane >> 2) & 1) == ((lane >> 4) & 1)) ? El<E>::ONE2 : 0u;
  return __builtin_bit_cast(bf16x8, u32x4{w, w, w, w});
}

// Probabilities of a 32x32 tile: p = 2^(s * scale - ref), packed in pairs to
// the element type (rounded toward zero) as the four P^T operands.
template <int E>
__device__ __forceinline__ void probs32(const f32x16 (&s)[2], float sl, float nref, u32x4 (&pk)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 8 * (t & 1) + 2 * k;
      pk[t][k] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[t >> 1][e], sl, nref)),
                               __builtin_amdgcn_exp2f(__builtin_fmaf(s[t >> 1][e + 1], sl, nref)));
    }
}

// Slot (within the stage) of element e of block sb for lane half h.
__device__ __forceinline__ int slot32(int sb, int e, int h) {
  return 32 * sb + 16 * (e >> 3) + 8 * h + 4 * ((e >> 2) & 1) + (e & 3);
}

// Rare branch: scores of slots at or past `valid` become -inf.  Wait states
// first, clear of the MFMAs that wrote s.
__device__ __forceinline__ void mask32(f32x16 (&s)[2], int valid, int h) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  int lim = valid;
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (slot32(sb, e, h) >= lim) s[sb][e] = -INFINITY;
}

__device__ __forceinline__ void mask16(f32x4& s, int valid, int slot0) {
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  int lim = valid - slot0;
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j >= lim) s[j] = -INFINITY;
}

// Exact path of a 32x32 tile (rare): column maximum of s * scale - ref over
// the stage (the lane's 32 slots and those of lane ^ 32), ref moved up to it
// (set, while the tile has seen no valid slot, `fresh`), the running sum and
// output scaled by 2^-(shift), and the probabilities recomputed.  Returns the
// column sum of the recomputed (rounded) probabilities.
template <int DB, int E>
__device__ __forceinline__ float renorm32(const f32x16 (&s)[2], float sl, int& fresh, float& ref, float& nref,
                                          float& l, f32x16 (&o)[DB], u32x4 (&pk)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float m = s[0][0];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = max2(m, s[sb][e]);
  {
    uint32_t a = __builtin_bit_cast(uint32_t, m), b = a;
    swap32(a, b);
    m = max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  }
  m = __builtin_fmaf(m, sl, nref);
  const bool first = fresh != 0;
  fresh = __builtin_amdgcn_readfirstlane((int)(first && __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0));
  const float shift = first ? (m == -INFINITY ? 0.0f : m) : fmaxf(m, 0.0f);
  // (one block of four accumulators, one k-step of probabilities at a
  // time: this branch runs while every value of the hot loop is live)
  if (!first) {
    const float alpha = __builtin_amdgcn_exp2f(-shift);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[db][4 * q4 + j] *= alpha;
      }
  }
  ref += shift;
  nref = -ref;
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 8 * (t & 1) + 2 * k;
      pk[t][k] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[t >> 1][e], sl, nref)),
                               __builtin_amdgcn_exp2f(__builtin_fmaf(s[t >> 1][e + 1], sl, nref)));
    }
    a = El<E>::dot_ones(pk[t][0], a);
    b = El<E>::dot_ones(pk[t][1], b);
    a = El<E>::dot_ones(pk[t][2], a);
    b = El<E>::dot_ones(pk[t][3], b);
  }
  __builtin_amdgcn_sched_barrier(0);
  float sum = a + b;
  {
    uint32_t x = __builtin_bit_cast(uint32_t, sum), y = x;
    swap32(x, y);
    sum = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
  }
  asm volatile("s_nop 3" ::: "memory");
  return sum;
}

// Exact path of a bfloat16 32x32 tile without the scores: the column's
// largest packed probability 2^e m (e its exponent field) fixes the integer
// shift k = e - 126 that brings it into [0.5, 1); the running sum and output
// are scaled by 2^-k, ref moves up by k and every packed probability is
// divided by 2^k exactly, by lowering its exponent field (a value that would
// fall below the normal range becomes 0: under 2^-126 of the new maximum).
// The result is what exp2 against the moved ref gives, truncated the same
// way, so the scores need not stay live past the softmax.  It cannot stand in
// for them when a probability overflowed (exponent field 255) or, on a tile
// with no state yet and valid slots in the stage, when the largest
// probability is under 2^-60 (smaller terms may have underflowed): then the
// wave sets `need` and the caller redoes the split with renorm32.
template <int DB>
__device__ __forceinline__ float renorm32pk(int& fresh, float& ref, float& nref, float& l, f32x16 (&o)[DB],
                                            u32x4 (&pk)[4], int valid, int& need) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, pk[0][0]);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, pk[t][k]));
  uint32_t mb = m.x > m.y ? m.x : m.y;
  {
    uint32_t a = mb, b = mb;
    swap32(a, b);
    mb = a > b ? a : b;
  }
  const int ex = (int)((mb >> 7) & 0xFF);
  const bool first = fresh != 0;
  if (__builtin_amdgcn_ballot_w64(ex == 0xFF || (first && valid > 0 && mb < 0x2180u)) != 0) {
    need = 1;   // the split is redone with the scores
    return 0.f;
  }
  // a column with no valid slot yet keeps the tile fresh (all slots masked)
  fresh = __builtin_amdgcn_readfirstlane((int)(first && __builtin_amdgcn_ballot_w64(mb == 0u) != 0));
  int shift = mb == 0u ? 0 : ex - 126;
  if (!first && shift < 0) shift = 0;
  if (!first) {
    const float alpha = __builtin_amdgcn_ldexpf(1.0f, -shift);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[db][4 * q4 + j] *= alpha;
      }
  }
  ref += (float)shift;
  nref = -ref;
  float a = 0.f, b = 0.f;
  const int sh7 = shift << 7;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = pk[t][k];
      const int lo0 = (int)(w & 0xFFFFu), hi0 = (int)(w >> 16);
      const int lo = lo0 - sh7, hi = hi0 - sh7;
      pk[t][k] = (uint32_t)((lo0 == 0 || lo < 0x80) ? 0 : lo) | ((uint32_t)((hi0 == 0 || hi < 0x80) ? 0 : hi) << 16);
    }
    a = El<0>::dot_ones(pk[t][0], a);
    b = El<0>::dot_ones(pk[t][1], b);
    a = El<0>::dot_ones(pk[t][2], a);
    b = El<0>::dot_ones(pk[t][3], b);
  }
  float sum = a + b;
  {
    uint32_t x = __builtin_bit_cast(uint32_t, sum), y = x;
    swap32(x, y);
    sum = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
  }
  asm volatile("s_nop 3" ::: "memory");
  return sum;
}

// The same for the tail's 16x16 block (4 slots per lane; a column's 16
// slots sit in lanes l, l ^ 16, l ^ 32, l ^ 48).  Returns the lane's sum.
template <int TDB, int E>
__device__ __forceinline__ float renorm16(const f32x4& s, float sl, int& fresh, float& ref, float& nref, float& l,
                                          f32x4 (&o)[TDB], u32x2& pk) {
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  float m = max2(max2(s[0], s[1]), max2(s[2], s[3]));
  m = __builtin_fmaf(lane_swap_max(m), sl, nref);
  const bool first = fresh != 0;
  fresh = __builtin_amdgcn_readfirstlane((int)(first && __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0));
  const float shift = first ? (m == -INFINITY ? 0.0f : m) : fmaxf(m, 0.0f);
  if (!first) {
    const float alpha = __builtin_amdgcn_exp2f(-shift);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < TDB; ++db) o[db] *= alpha;
  }
  ref += shift;
  nref = -ref;
  pk[0] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[0], sl, nref)),
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[1], sl, nref)));
  pk[1] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(s[2], sl, nref)),
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[3], sl, nref)));
  const float lt = El<E>::dot_ones(pk[1], El<E>::dot_ones(pk[0], 0.f));
  asm volatile("s_nop 3" ::: "memory");
  return lt;
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Barrier that first waits for the wave's LDS reads: after it, other waves'
// direct-to-LDS loads may refill the ring slots those reads came from.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most `a` stages (LPW loads each) of the wave's direct-to-LDS
// loads are outstanding (a <= A; vmcnt takes an immediate).
template <int LPW, int A>
__device__ __forceinline__ void wait_ahead(int a) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (a >= A)
      wait_vmcnt<A * LPW>();
    else
      wait_ahead<LPW, A - 1>(a);
  }
}

// FUSED: launched by kvc_run_append (p.fused = 1): units whose entry z is
// nonzero are read from the caller's k and v.
template <int D, int E, bool TAIL, bool FUSED>
__global__ __launch_bounds__(64 * KVC_ATTN32_WAVES, 1) void attn32_kernel(AttnParams p) {
  using S = Shape32<D>;
  using MM = M32<E>;
  constexpr int NW = KVC_ATTN32_WAVES;
  constexpr int KS = S::KS, DB = S::DB, TKS = S::TKS, TDB = S::TDB, LPW = S::LPW, NST = S::NSTAGE;
  // LDS: the ring of K/V stages and the split's unit entries.  Before the
  // loop the last three ring slots stage the query operands: per wave its
  // tile (and, for the tail waves, a copy of the tail), row-major.
  constexpr int QW = (S::QT + (TAIL ? S::TQ : 0)) * 1024;
  static_assert(NW * QW <= 3 * S::STAGE, "query staging fits three ring slots");
  constexpr int P0 = NST - 3;   // stages loaded before the query operands are read
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NST * S::STAGE];
  __shared__ __attribute__((aligned(1024))) int4 elds[KVC_MAX_SPLIT_STAGES];
  // set when a wave needs the split redone with the exact path on the scores
  __shared__ int xflag[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 31, h = lane >> 5;       // 32x32 layouts: query column, lane half
  const int r16 = lane & 15, g4 = lane >> 4;    // 16x16 layouts
  // Waves w and w + 4 share a SIMD.  A lead wave (w < 4) does QK, softmax
  // and P.V of stage s in iteration s; its lag partner does the softmax and
  // P.V of stage s - 1, then QK of stage s: while one runs MFMAs the other
  // runs the vector unit.  The lead waves also share the tail.
  const bool lead = wv < KVC_TAIL_WAVES;

  // XCD-aware item order: work-groups go round-robin over the 8 XCDs; each
  // XCD takes a contiguous item range, so one head's splits share an L2.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * p.items_per_xcd + (bid >> 3);
  if (item >= p.num_items) return;

  const kvc_dev_stream st = stream_of_item(p, item);

  int local = item - st.item0;
  const int grp = local % st.n_group;
  local /= st.n_group;
  const int split = local % st.n_split;
  const int hd = local / st.n_split;

  // tiles of 32 rows of this group (one per wave), and the tail (16 rows) if
  // this group has it
  const int t_lo = grp * st.n_t32 / st.n_group;
  const int t_hi = (grp + 1) * st.n_t32 / st.n_group;
  const int ntile = t_hi - t_lo;
  const int tile = t_lo + wv;
  const bool has_tail = TAIL && st.tail != 0 && grp == st.n_group - 1;
  const int u0 = split * st.n_units / st.n_split;
  const int u1 = (split + 1) * st.n_units / st.n_split;
  const int nstage = u1 - u0;
  const int H = p.num_heads;
  const uint32_t slot_bytes = (uint32_t)H * D * 2;
  const int32_t* units = p.plan + st.unit0 + KVC_UNIT_INTS * u0;
  const uint64_t head_off = (uint64_t)hd * D * 2;
  const float sl = p.scale_log2;

  // Unit entries (the host planner resolved pages, chunks and valid
  // lengths): those of the first stages by scalar loads, ahead of every
  // other memory operation; all of them copied to LDS by direct loads for the
  // stage loop, which then issues no global memory operation besides its
  // direct-to-LDS loads (whose completion it counts with vmcnt).
  int4 e_first[P0];
#pragma unroll
  for (int i = 0; i < P0; ++i)
    e_first[i] = i < nstage ? int4{units[KVC_UNIT_INTS * i], units[KVC_UNIT_INTS * i + 1],
                                   FUSED ? units[KVC_UNIT_INTS * i + 2] : 0, 0}
                            : int4{0, KVC_KV_TILE, 0, 0};
  auto uniform_entry = [](const int4& e) {
    return int4{__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                FUSED ? __builtin_amdgcn_readfirstlane(e.z) : 0, 0};
  };
  auto stage_entry = [&](int i) { return uniform_entry(elds[i]); };

  // ---- direct global -> LDS loads of one stage (K rows, then V rows) ----
  // Load instruction j of the wave fills 1 KiB at LDS byte 1024 * (wave *
  // LPW + j) of the stage, lane l writing [16 l, 16 l + 16); the lane fetches
  // the logical chunk the swizzle places there.
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  const uint64_t v_half = (uint64_t)p.page_size * slot_bytes;
  // Fused append: units of the step's own rows (entry z = 1 + input row)
  // are read from the caller's k and v of the item's stream, whose rows have
  // the pool's row layout; V is vin - kin bytes past K there.
  const uint8_t* kin = nullptr;
  uint64_t vin_delta = 0;
  if constexpr (FUSED) {
    const void* kb = p.kin[0];
    const void* vb = p.vin[0];
#pragma unroll
    for (int i = 1; i < KVC_ARG_STREAMS; ++i)
      if (i < p.num_streams && item >= p.recs[i].item0) {
        kb = p.kin[i];
        vb = p.vin[i];
      }
    kin = static_cast<const uint8_t*>(kb);
    vin_delta = (uint64_t)(uintptr_t)vb - (uint64_t)(uintptr_t)kb;
  }
  // Load instruction i of a stage (K: i < LOADS / 2, V: the rest) covers
  // rows RPL (i % (LOADS / 2)) .. + RPL - 1 of its half; lane l writes chunk
  // l % CPR of row RPL (i % ...) + l / CPR.  The swizzle depends on row bits
  // 1-3.  With D = 32 (RPL = 16) they all come from l / CPR; with D = 64
  // (RPL = 8) bit 3 is the parity of the load's row block, which is that of
  // the wave's load index j (LPW and LOADS / 2 are even).  So one per-lane
  // offset per block parity serves every load, and the row offset
  // RPL (i % ...) joins the (scalar) base address.
  constexpr int CPR = S::ROW_BYTES / 16, RPL = 1024 / S::ROW_BYTES;
  static_assert(RPL % 16 == 0 || (RPL == 8 && LPW % 2 == 0 && (S::LOADS / 2) % 2 == 0), "load row blocks");
  const int lrow0 = lane / CPR;
  const uint32_t lofs0 = (uint32_t)lrow0 * slot_bytes + (uint32_t)(((lane % CPR) ^ swz32<D>(lrow0)) << 4);
  const uint32_t lofs1 =
      RPL == 8 ? (uint32_t)lrow0 * slot_bytes + (uint32_t)(((lane % CPR) ^ swz32<D>(lrow0 + 8)) << 4) : lofs0;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  // per load j of this wave: its first row in the unit, its half (all the
  // wave's loads are K loads or all V loads) and its LDS offset in a stage
  // (uniform)
  static_assert((S::LOADS / 2) % LPW == 0, "a wave's loads stay in one half");
  const bool wave_v = wv * LPW >= S::LOADS / 2;
  uint32_t jlds[LPW];
  int jrow[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int inst = wv * LPW + j;
    const int kv = inst >= S::LOADS / 2 ? 1 : 0;
    const int blk = inst - kv * (S::LOADS / 2);
    jrow[j] = RPL * blk;
    jlds[j] = (uint32_t)(kv * S::HALF + blk * 1024);
  }
  // load j of a stage whose unit starts at ubase, into the ring slot at LDS
  // byte `slot`: rows past the valid count (a partial stage) re-read the last
  // valid row.  The offset is an unsigned 32-bit addend of the scalar base
  // (the unit's first row of the K or V half), so rows are measured from the
  // unit's first row, never below it.
  auto issue_e = [&](int sidx, int4 e) {
    const bool in = FUSED && e.z != 0;
    const uint8_t* kbase = in ? kin + (uint64_t)(uint32_t)(e.z - 1) * slot_bytes
                              : pool + (uint64_t)(uint32_t)e.x * slot_bytes;
    const uint8_t* ubase = kbase + head_off + (wave_v ? (in ? vin_delta : v_half) : 0);
    const uint32_t slot = ring_lds + (uint32_t)(sidx % NST) * S::STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const uint32_t o =
          ((j & 1) ? lofs1 : lofs0) + (uint32_t)(min(jrow[j] + lrow0, e.y - 1) - lrow0) * slot_bytes;
      load_lds16(ubase, o, slot + jlds[j]);
    }
  };

  // ---- prologue loads, in the order the vmcnt accounting assumes ----
  // (1) query rows (RPL per load, row-major) into the staging slots; rows
  // past the stream's queries repeat its last row (their columns are never
  // stored)
  const uint32_t qlds = ring_lds + (uint32_t)((NST - 3) * S::STAGE + wv * QW);
  const uint8_t* qsrc = static_cast<const uint8_t*>(p.q) + ((size_t)st.q_row0 * H + hd) * D * 2;
  auto q_dma = [&](int row0, int nload, uint32_t lds0) {
    const int r0 = min(row0, st.n_q - 1);
#pragma unroll
    for (int i = 0; i < nload; ++i) {
      const int row = min(row0 + RPL * i + lrow0, st.n_q - 1);
      load_lds16(qsrc + (size_t)r0 * slot_bytes, (uint32_t)(row - r0) * slot_bytes + (uint32_t)((lane % CPR) << 4),
                 lds0 + (uint32_t)(i * 1024));
    }
  };
  q_dma(32 * tile, S::QT, qlds);
  if constexpr (TAIL)
    if (lead) q_dma(32 * st.n_t32, S::TQ, qlds + S::QT * 1024);
  // (2) unit entries, 64 per load, by the waves in turn (lanes past the
  // split's count repeat its last entry)
  {
    const uint32_t elds_lds = __builtin_amdgcn_readfirstlane(lds_addr(elds));
    const int nblk = (nstage + 63) / 64;
    for (int b = wv; b < nblk; b += NW)
      load_lds16(units, (uint32_t)min(64 * b + lane, nstage - 1) * 16, elds_lds + (uint32_t)(b * 1024));
  }
  // (3) the first stages
  const int pre = min(nstage, P0);
#pragma unroll
  for (int i = 0; i < P0; ++i)
    if (i < pre) issue_e(i, e_first[i]);

  // ---- LDS operand offsets (per lane; stage base added at the read) ----
  uint32_t kofs[KS];          // K rows (A of S^T): row kperm(n) of each 32-slot block, chunk 2ks + h
  {
    const int row = kperm(n);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kofs[ks] = (uint32_t)(row * S::ROW_BYTES + (((2 * ks + h) ^ swz32<D>(row)) << 4));
  }
  uint32_t vofs[DB][2];       // V^T (A of O^T) by transposing reads: k-step 0; + 16 rows per k-step
  {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 8 * (g >> 1) + 4 * rr + (s >> 2);
        const int c = 4 * db + 2 * (g & 1) + ((s & 3) >> 1);
        vofs[db][rr] = (uint32_t)(S::HALF + row * S::ROW_BYTES + ((c ^ swz32<D>(row)) << 4) + 8 * (s & 1));
      }
  }
  uint32_t tkofs[TKS], tvofs[TDB];   // tail (lead waves): K rows 16w + r16; V^T rows 16w + 4 g4 + s / 4
  if constexpr (TAIL) {
    const int row = 16 * (wv & 3) + r16;
#pragma unroll
    for (int k = 0; k < TKS; ++k)
      tkofs[k] = (uint32_t)(row * S::ROW_BYTES + (((4 * k + g4) ^ swz32<D>(row)) << 4));
    const int s = lane & 15;
    const int vrow = 16 * (wv & 3) + 4 * g4 + (s >> 2);
#pragma unroll
    for (int db = 0; db < TDB; ++db) {
      const int c = 2 * db + ((s & 3) >> 1);
      tvofs[db] = (uint32_t)(S::HALF + vrow * S::ROW_BYTES + ((c ^ swz32<D>(vrow)) << 4) + 8 * (s & 1));
    }
  }

  bf16x8 kop[2][KS], vop[4][DB];
  bf16x8 tk[TKS];
  bf16x4 tv[TDB];
  auto read_k = [&](int sidx) {
    const uint8_t* b = ring + (sidx % NST) * S::STAGE;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[sb][ks] = *reinterpret_cast<const bf16x8*>(b + kofs[ks] + 32 * sb * S::ROW_BYTES);
  };
  auto read_v = [&](int sidx) {
    const uint8_t* b = ring + (sidx % NST) * S::STAGE;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 x0 = ds_read_tr16(b + vofs[db][0] + 16 * t * S::ROW_BYTES);
        const i16x4 x1 = ds_read_tr16(b + vofs[db][1] + 16 * t * S::ROW_BYTES);
        vop[t][db] = __builtin_bit_cast(
            bf16x8, (short __attribute__((ext_vector_type(8)))){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
      }
  };
  auto read_tail = [&](int sidx) {
    const uint8_t* b = ring + (sidx % NST) * S::STAGE;
#pragma unroll
    for (int k = 0; k < TKS; ++k) tk[k] = *reinterpret_cast<const bf16x8*>(b + tkofs[k]);
#pragma unroll
    for (int db = 0; db < TDB; ++db) tv[db] = __builtin_bit_cast(bf16x4, ds_read_tr16(b + tvofs[db]));
  };

  // ---- softmax state of the wave's tile and (lead waves) of its tail block:
  // ref (log2 units) and its negation, running sum, fresh (no valid slot
  // seen yet) ----
  float ref = 0.f, nref = 0.f, l = 0.f, refT = 0.f, nrefT = 0.f, lT = 0.f;
  int fresh = 1, freshT = 1;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  f32x4 oT[TDB];
#pragma unroll
  for (int db = 0; db < TDB; ++db) oT[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8 mask = rowsum_mask<E>(lane);
  f32x16 sc[2];
  u32x4 pk[4];
  f32x4 sT;
  u32x2 pT = u32x2{0u, 0u};

  // the tile's probabilities in 16 chunks (chunk c: P^T operand t = c / 4,
  // pair c % 4), software-pipelined over three steps so that each result is
  // used one step after it was computed: step c packs chunk c-1, takes exp2
  // of chunk c and scales chunk c+1
  auto softmax = [&]() {
    float f0, f1, x0 = 0.f, x1 = 0.f;
    auto scale = [&](int c) {
      const int t = c >> 2, e = 8 * (t & 1) + 2 * (c & 3);
      f0 = __builtin_fmaf(sc[t >> 1][e], sl, nref);
      f1 = __builtin_fmaf(sc[t >> 1][e + 1], sl, nref);
    };
    scale(0);
#pragma unroll
    for (int c = 0; c <= 16; ++c) {
      if (c > 0) pk[(c - 1) >> 2][(c - 1) & 3] = El<E>::pack_p(x0, x1);
      if (c < 16) {
        x0 = __builtin_amdgcn_exp2f(f0);
        x1 = __builtin_amdgcn_exp2f(f1);
      }
      if (c + 1 < 16) scale(c + 1);
    }
  };
  auto rowsum = [&]() {
    f32x4 r = El<E>::mfma(mask, __builtin_bit_cast(bf16x8, pk[0]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int t = 1; t < 4; ++t) r = El<E>::mfma(mask, __builtin_bit_cast(bf16x8, pk[t]), r);
    return r;
  };
  // lazy check of the tile (column sums of the probabilities with the current
  // ref; the exact path when a sum is too large or the tile is fresh)
  // (bfloat16, first pass: the exact path from the packed probabilities, so
  // that the scores die with the softmax; the pass with `exact` set, and
  // float16, rebase from the scores)
  int need_exact = 0;
  auto check = [&](const f32x4& rs, int vld, auto exact_tag) {
    constexpr bool exact = decltype(exact_tag)::value;
    float cs = rs[0];
    if (__builtin_expect(fresh || __builtin_amdgcn_ballot_w64(sum_exceeds(cs, LAZY_COL_LIMIT)), 0)) {
      if constexpr (E == 0 && !exact)
        cs = renorm32pk<DB>(fresh, ref, nref, l, o, pk, vld, need_exact);
      else
        cs = renorm32<DB, E>(sc, sl, fresh, ref, nref, l, o, pk);
    }
    l += cs;
  };
  bf16x8 qv[KS], qT[TKS];
  auto qk = [&]() {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sc[sb] = MM::mfma32(kop[sb][0], qv[0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) sc[sb] = MM::mfma32(kop[sb][ks], qv[ks], sc[sb]);
    }
  };
  auto pv = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = MM::mfma32(vop[t][db], __builtin_bit_cast(bf16x8, pk[t]), o[db]);
  };
  // ---- prologue: query operands and stage 0 ----
  if (tid == 0) xflag[0] = 0;         // published by the barrier below
  wait_ahead<LPW, P0 - 1>(pre - 1);   // queries, entries and stage 0 landed (own loads)
  block_barrier();                    // ... and everyone's
  {
    // tile: lane (n, h) holds q[row n][16 ks + 8h .. + 8); tail: lane (r16,
    // g4) holds q[row r16][32 k + 8 g4 .. + 8)
    const uint8_t* qw = ring + (NST - 3) * S::STAGE + wv * QW;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qv[ks] = *reinterpret_cast<const bf16x8*>(qw + n * S::ROW_BYTES + (2 * ks + h) * 16);
    if constexpr (TAIL) {
#pragma unroll
      for (int k = 0; k < TKS; ++k)
        qT[k] = *reinterpret_cast<const bf16x8*>(qw + S::QT * 1024 + r16 * S::ROW_BYTES + (4 * k + g4) * 16);
    }
  }
  // every wave has its query operands: the staging slots take stages P0 ..
  ring_barrier();
  for (int i = P0; i < min(nstage, NST - 1); ++i) issue_e(i, stage_entry(i));
  // the lag waves start with "stage -1": all slots masked, zero operands; its
  // check takes the exact path and leaves the tile fresh and empty
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[sb][e] = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int db = 0; db < DB; ++db) vop[t][db] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

  // ---- stage loop: iteration s consumes ring slot s, published by the
  // barrier at its top, and refills the slot of stage s - 1 with stage
  // s + NST - 1 (two loops, with and without those loads) ----
  int4 e_next = elds[min(NST - 1, KVC_MAX_SPLIT_STAGES - 1)];
  int4 e_cur = elds[0];
  int valid_prev = 0;   // lag waves: valid slots of stage s - 1 (stage -1: none)
  auto stage_body = [&](int s, auto issue_tag, auto lead_tag, auto exact_tag) {
    constexpr bool do_issue = decltype(issue_tag)::value;
    constexpr bool is_lead = decltype(lead_tag)::value;
    wait_ahead<LPW, NST - 2>(min(nstage - 1 - s, NST - 2));
    ring_barrier();
    // the refill of the slot that stage s - 1 held (every wave has passed
    // the barrier, so none reads it any more) is issued after this
    // iteration's QK MFMAs: right after the barrier all 8 waves would queue
    // their loads at once
    const int4 e_iss = uniform_entry(e_next);
    const int valid = __builtin_amdgcn_readfirstlane(e_cur.y);
    e_cur = elds[min(s + 1, KVC_MAX_SPLIT_STAGES - 1)];
    e_next = elds[min(s + NST, KVC_MAX_SPLIT_STAGES - 1)];
    if constexpr (is_lead) {
      read_k(s);
      read_v(s);
      if constexpr (TAIL) read_tail(s);
      qk();
      if constexpr (do_issue) issue_e(s + NST - 1, e_iss);
      if constexpr (TAIL) {
        sT = El<E>::mfma(tk[0], qT[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int k = 1; k < TKS; ++k) sT = El<E>::mfma(tk[k], qT[k], sT);
      }
      if (__builtin_expect(valid < KVC_KV_TILE, 0)) {
        mask32(sc, valid, h);
        if constexpr (TAIL) mask16(sT, valid, 16 * wv + 4 * g4);
      }
      softmax();
      const f32x4 rs = rowsum();
      if constexpr (TAIL) {
        pT[0] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(sT[0], sl, nrefT)),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(sT[1], sl, nrefT)));
        pT[1] = El<E>::pack_p(__builtin_amdgcn_exp2f(__builtin_fmaf(sT[2], sl, nrefT)),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(sT[3], sl, nrefT)));
        float lt = El<E>::dot_ones(pT[1], El<E>::dot_ones(pT[0], 0.f));
        if (__builtin_expect(freshT || __builtin_amdgcn_ballot_w64(sum_exceeds(lt, LAZY_SUM_LIMIT)), 0))
          lt = renorm16<TDB, E>(sT, sl, freshT, refT, nrefT, lT, oT, pT);
        lT += lt;
      }
      check(rs, valid, exact_tag);
      pv();
      if constexpr (TAIL) {
#pragma unroll
        for (int db = 0; db < TDB; ++db) oT[db] = MM::mfma16x16(tv[db], __builtin_bit_cast(bf16x4, pT), oT[db]);
      }
    } else {
      // stage s - 1: scores in sc, V in vop
      softmax();
      check(rowsum(), valid_prev, exact_tag);
      valid_prev = valid;
      pv();
      // stage s: V into vop for the next iteration, scores into sc
      read_k(s);
      read_v(s);
      qk();
      if constexpr (do_issue) issue_e(s + NST - 1, e_iss);
      if (__builtin_expect(valid < KVC_KV_TILE, 0)) mask32(sc, valid, h);
    }
  };
  // one loop per role: each keeps its loop-carried accumulators in its own
  // registers (a shared loop with a role branch inside made the compiler
  // copy the output accumulators between the branches every stage)
  // the lead waves issue ahead of their lag partners when both are ready
  // (measured: 0.17 us shorter launches; the other way round, 1.8 us longer)
  if (lead) __builtin_amdgcn_s_setprio(2);
  auto pass = [&](auto exact_tag) {
    if (lead) {
      int s = 0;
      for (; s + NST - 1 < nstage; ++s) stage_body(s, Flag<true>{}, Flag<true>{}, exact_tag);
      for (; s < nstage; ++s) stage_body(s, Flag<false>{}, Flag<true>{}, exact_tag);
    } else {
      int s = 0;
      for (; s + NST - 1 < nstage; ++s) stage_body(s, Flag<true>{}, Flag<false>{}, exact_tag);
      for (; s < nstage; ++s) stage_body(s, Flag<false>{}, Flag<false>{}, exact_tag);
    }
    // ---- drain: the lag waves' last stage ----
    if (!lead) {
      softmax();
      check(rowsum(), valid_prev, exact_tag);
      pv();
    }
  };
  pass(Flag<false>{});
  if constexpr (E == 0) {
    // A wave whose packed probabilities could not stand in for the scores
    // (an overflow, or a first stage far below the reference) asks for the
    // split again with the exact path on the scores; the work-group decides
    // together (every wave is done with the ring at the barrier).
    if (need_exact && lane == 0) xflag[0] = 1;
    ring_barrier();
    if (__builtin_amdgcn_readfirstlane(xflag[0])) {
      ref = nref = l = refT = nrefT = lT = 0.f;
      fresh = freshT = 1;
      valid_prev = 0;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
#pragma unroll
      for (int db = 0; db < TDB; ++db) oT[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[sb][e] = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) vop[t][db] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      e_next = elds[min(NST - 1, KVC_MAX_SPLIT_STAGES - 1)];
      e_cur = elds[0];
      for (int i = 0; i < min(nstage, NST - 1); ++i) issue_e(i, stage_entry(i));
      pass(Flag<true>{});
    }
  }
  // the epilogue reads the accumulators the last MFMAs wrote
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- epilogue ----
  // lane (n, h) holds O^T[32 db + 8 i + 4 h + j][query n] in element 4 i + j
  // of block db.
  if (wv < ntile) {
    const float inv = 1.0f / l;
    const int row = 32 * tile + n;
    if (st.n_split > 1) {
      // normalised partial output (a convex combination of V rows, rounded
      // to the element type) in the accumulator's lane order, and its
      // log-sum-exp; rows past the stream's queries are stored too (never
      // merged).  Non-temporal stores: the merge launch reads them once,
      // and they leave the L2 before the launch ends.
      const size_t pt = ((size_t)split * H + hd) * p.tiles_cap + st.q_tile0 + tile;
      uint16_t* po = static_cast<uint16_t*>(p.part_o) + pt * (size_t)(DB * 4 * 256) + lane * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = f32x4{o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]} * inv;
          __builtin_nontemporal_store(El<E>::cvt4(v), reinterpret_cast<u32x2*>(po + (db * 4 + i) * 256));
        }
      if (h == 0) __builtin_nontemporal_store(ref + __log2f(l), p.part_lse + pt * 32 + n);
    } else if (row < st.n_q) {
      uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)(st.q_row0 + row) * H + hd) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = f32x4{o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]} * inv;
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * i + 4 * h) = El<E>::cvt4(v);
        }
    }
  }

  if constexpr (TAIL) {
    if (has_tail) {
      // merge the lead waves' states of the tail (weights 2^(ref_w - max
      // ref)); a wave whose slots were all masked has l = 0
      constexpr int NV = TDB * 4 + 2;
      float* xs = reinterpret_cast<float*>(ring);
      const float lsum_w = lane_swap_sum(lT);
      __syncthreads();   // every wave is done with the ring
      if (lead) {
#pragma unroll
        for (int db = 0; db < TDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) xs[(wv * 64 + lane) * NV + 4 * db + j] = oT[db][j];
        xs[(wv * 64 + lane) * NV + TDB * 4] = lsum_w > 0.0f ? refT : -INFINITY;
        xs[(wv * 64 + lane) * NV + TDB * 4 + 1] = lsum_w;
      }
      __syncthreads();
      if (wv == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < KVC_TAIL_WAVES; ++w) M = fmaxf(M, xs[(w * 64 + lane) * NV + TDB * 4]);
        float lsum = 0.f;
        f32x4 ot[TDB];
#pragma unroll
        for (int db = 0; db < TDB; ++db) ot[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < KVC_TAIL_WAVES; ++w) {
          const float* x = xs + (w * 64 + lane) * NV;
          const float wt = __builtin_amdgcn_exp2f(x[TDB * 4] - M);
          lsum += wt * x[TDB * 4 + 1];
#pragma unroll
          for (int db = 0; db < TDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) ot[db][j] += wt * x[4 * db + j];
        }
        const float inv = 1.0f / lsum;
        // lane (r16, g4) holds O^T[16 db + 4 g4 + j][tail query r16]
        if (st.n_split > 1) {
          // stored as rows 0-15 of the 32-row tile after the full ones, in
          // the 32x32 accumulator lane order the merge reads
          const size_t pt = ((size_t)split * H + hd) * p.tiles_cap + st.q_tile0 + st.n_t32;
          uint16_t* po = static_cast<uint16_t*>(p.part_o) + pt * (size_t)(DB * 4 * 256);
#pragma unroll
          for (int db = 0; db < TDB; ++db) {
            const int d = 16 * db + 4 * g4;
            const int b32 = d >> 5, i = (d & 31) >> 3, hh = (d >> 2) & 1;
            __builtin_nontemporal_store(El<E>::cvt4(ot[db] * inv),
                                        reinterpret_cast<u32x2*>(po + (b32 * 4 + i) * 256 + (32 * hh + r16) * 4));
          }
          if (g4 == 0) __builtin_nontemporal_store(M + __log2f(lsum), p.part_lse + pt * 32 + r16);
        } else {
          const int row = 32 * st.n_t32 + r16;
          if (row < st.n_q) {
            uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)(st.q_row0 + row) * H + hd) * D;
#pragma unroll
            for (int db = 0; db < TDB; ++db)
              *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g4) = El<E>::cvt4(ot[db] * inv);
          }
        }
      }
    }
  }
}

template <int E, bool TAIL, bool FUSED>
int launch32_etf(const AttnParams& p, int32_t grid, hipStream_t hs) {
  switch (p.head_dim) {
    case 32:
      hipLaunchKernelGGL((attn32_kernel<32, E, TAIL, FUSED>), dim3(grid), dim3(64 * KVC_ATTN32_WAVES), 0, hs, p);
      break;
    case 64:
      hipLaunchKernelGGL((attn32_kernel<64, E, TAIL, FUSED>), dim3(grid), dim3(64 * KVC_ATTN32_WAVES), 0, hs, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int E, bool TAIL>
int launch32_et(const AttnParams& p, int32_t grid, hipStream_t hs) {
  return p.fused ? launch32_etf<E, TAIL, true>(p, grid, hs) : launch32_etf<E, TAIL, false>(p, grid, hs);
}

}  // namespace

int launch_attention32(const AttnParams& p, int32_t grid, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  if (p.dtype == 0) return p.shared_tile ? launch32_et<0, true>(p, grid, hs) : launch32_et<0, false>(p, grid, hs);
  if (p.dtype == 1) return p.shared_tile ? launch32_et<1, true>(p, grid, hs) : launch32_et<1, false>(p, grid, hs);
  return (int)hipErrorInvalidValue;
}

}  // namespace kvc
