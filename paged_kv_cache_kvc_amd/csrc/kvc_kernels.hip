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

#include "kvc_kernels.h"

namespace kvc {

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.div = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shr = s;
  const uint64_t m = ((1ull << (32 + s)) + d - 1) / d;
  f.mul = (uint32_t)(m - (1ull << 32));
  return f;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = KVC_KV_TILE;

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.mul) + n) >> f.shr;
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
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
  const int chunks = p.row_elems >> 3;   // 16-byte chunks per row; H*D is a multiple of 32
  const size_t row_off = (size_t)r * p.row_elems;
  const u32x4* sk = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.k) + row_off);
  const u32x4* sv = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.v) + row_off);
  uint16_t* pool = static_cast<uint16_t*>(p.pool);
  u32x4* dk = reinterpret_cast<u32x4*>(pool + (((size_t)page * 2 + 0) * p.page_size + slot) * p.row_elems);
  u32x4* dv = reinterpret_cast<u32x4*>(pool + (((size_t)page * 2 + 1) * p.page_size + slot) * p.row_elems);
  for (int i = threadIdx.x; i < 2 * chunks; i += blockDim.x) {
    if (i < chunks)
      dk[i] = sk[i];
    else
      dv[i - chunks] = sv[i - chunks];
  }
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

// 16-byte chunk swizzle inside a K/V row of LDS: keeps the MFMA operand reads
// of 16 rows spread over the banks.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 1) | (((row >> 3) & 3) << 1); }

// The ring of stages is filled by direct global->LDS loads that the kernel
// issues, waits for and publishes itself: the compiler would otherwise treat
// every LDS read as depending on every load in flight and drain the ring at
// each barrier.  Completion is tracked with vmcnt (vector memory operations
// retire in issue order), then a barrier makes a stage visible to all waves.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes from base + offset (per lane) to LDS byte address
// lds_base + 16 * lane.  base is wave-uniform (scalar registers).
__device__ __forceinline__ void load_lds16(const void* base, uint32_t offset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"(base),
               "s"(lds_base)
               : "memory", "m0");
}

// Maximum of scores (never NaN: masked slots are -inf).  Written with the
// compiler's own max so that its hazard tracking sees the MFMA results these
// read (an opaque instruction reading an MFMA accumulator too early would see
// a partially written register).
__device__ __forceinline__ float max3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }
__device__ __forceinline__ float max2(float a, float b) { return __builtin_fmaxf(a, b); }

__device__ __forceinline__ uint32_t lds_addr(const void* generic) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)generic;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i16x4 ds_read_tr16(const uint8_t* lds_generic) {
  const lds_i16x4* p = (const lds_i16x4*)(__attribute__((address_space(3))) const uint8_t*)lds_generic;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// Exchange with the lane 32 (or 16) apart: after the swap, each lane holds
// its own value and its partner's in (a, b).  Issued directly because the
// compiler builtin's second result is not usable.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// max / sum over lanes l, l^16, l^32, l^48: the four lane groups that hold
// one query column of an MFMA accumulator
__device__ __forceinline__ float lane_swap_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float lane_swap_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Rescale threshold of the running maximum, in log2 units of the scaled
// scores: probabilities up to 2^8 are kept without renormalising.
constexpr float RESCALE_LOG2 = 8.0f;

// Work of one query tile over one 64-slot stage, in three parts so that
// the next tile's QK^T MFMAs can be issued before this tile's softmax (the
// matrix core then runs while the vector unit computes exponentials).
template <int D>
struct TileOps {
  using S = Shape<D>;

  // S^T[64 kv x 16 q] = K Q^T for the four 16-kv blocks of the stage
  static __device__ __forceinline__ void qk(const bf16x8 (&kop)[4][S::KSTEPS], const bf16x8 (&q)[S::KSTEPS],
                                            f32x4 (&sacc)[4]) {
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi) {
      sacc[kbi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks)
        sacc[kbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kbi][ks], q[ks], sacc[kbi], 0, 0, 0);
    }
  }

  // Online softmax of one tile's stage scores (fp32): mask slots past
  // `valid`, column max over the 64 kv, renormalise only when a column's
  // maximum grew by more than 2^RESCALE_LOG2, then p = 2^(s*sl - m) rounded
  // to bf16 into the P^T operand, and the row sums of those bf16 values.
  static __device__ __forceinline__ void softmax(f32x4 (&sacc)[4], int valid, int g4, float sl, float& mb, float& l,
                                                 f32x4 (&o)[S::DBLK], bf16x8 (&pb)[2]) {
    if (valid < KT) {
#pragma unroll
      for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (32 * (kbi >> 1) + 8 * g4 + 4 * (kbi & 1) + i >= valid) sacc[kbi][i] = -INFINITY;
    }
    float mx = max3(sacc[0][0], sacc[0][1], sacc[0][2]);
    mx = max3(mx, sacc[0][3], sacc[1][0]);
    mx = max3(mx, sacc[1][1], sacc[1][2]);
    mx = max3(mx, sacc[1][3], sacc[2][0]);
    mx = max3(mx, sacc[2][1], sacc[2][2]);
    mx = max3(mx, sacc[2][3], sacc[3][0]);
    mx = max3(mx, sacc[3][1], sacc[3][2]);
    mx = max2(mx, sacc[3][3]);
    mx = lane_swap_max(mx) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > mb + RESCALE_LOG2)) {
      const float nm = fmaxf(mb, mx);
      const float alpha = __builtin_amdgcn_exp2f(mb - nm);
      mb = nm;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) o[db] *= alpha;
    }
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pb[kbi >> 1][4 * (kbi & 1) + i] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbi][i], sl, -mb));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[pp][2 * j], pb[pp][2 * j + 1]}, ones, l, false);
  }

  // O^T[D x 16 q] += V^T P^T
  static __device__ __forceinline__ void pv(const bf16x8 (&vop)[S::DBLK][2], const bf16x8 (&pb)[2],
                                            f32x4 (&o)[S::DBLK]) {
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db][pp], pb[pp], o[db], 0, 0, 0);
  }

  // The shared tile on one 16-kv block BLK of the stage (BLK = 2*pair +
  // half), in two parts like the own tiles: QK^T first (issued one tile
  // ahead of its use), then softmax over its 4 scores per lane and P.V with
  // the other half of the pair's P^T operand zero.  A block whose slots are
  // all past the end of the stage is skipped.
  template <int BLK>
  static __device__ __forceinline__ bool block_live(int valid) {
    return 32 * (BLK >> 1) + 4 * (BLK & 1) < valid;
  }
  template <int BLK>
  static __device__ __forceinline__ f32x4 shared_qk(const bf16x8 (&kop)[4][S::KSTEPS], const bf16x8 (&q)[S::KSTEPS]) {
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[BLK][ks], q[ks], sc, 0, 0, 0);
    return sc;
  }
  template <int BLK>
  static __device__ __forceinline__ void shared_rest(f32x4 sc, const bf16x8 (&vop)[S::DBLK][2], int valid, int g4,
                                                     float sl, float& mb, float& l, f32x4 (&o)[S::DBLK]) {
    constexpr int PP = BLK >> 1, TT = BLK & 1;
    if (valid < KT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (32 * PP + 8 * g4 + 4 * TT + i >= valid) sc[i] = -INFINITY;
    }
    float mx = max2(max3(sc[0], sc[1], sc[2]), sc[3]);
    mx = lane_swap_max(mx) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > mb + RESCALE_LOG2)) {
      const float nm = fmaxf(mb, mx);
      const float alpha = __builtin_amdgcn_exp2f(mb - nm);
      mb = nm;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) o[db] *= alpha;
    }
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = (__bf16)0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[4 * TT + i] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], sl, -mb));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[4 * TT], pb[4 * TT + 1]}, ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[4 * TT + 2], pb[4 * TT + 3]}, ones, l, false);
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db][PP], pb, o[db], 0, 0, 0);
  }
};

// Attention over one KV split for one head and one query group.  The group's
// query tiles are spread over the 4 waves: each wave owns up to QTW tiles
// (t_lo + wave + 4k); when the group has 4m+1 tiles, the last one is shared:
// every wave processes one 16-kv block of it in every stage, and the four
// partial softmax states are merged through LDS at the end.  Every SIMD thus
// carries the same MFMA work per stage.
template <int D, int QTW>
__global__ __launch_bounds__(256, (D <= 64 ? 2 : 1)) void attn_kernel(AttnParams p) {
  using S = Shape<D>;
  using T = TileOps<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S::NSTAGE * S::STAGE_BYTES];
  // per stage of this split: byte offset of its first K row in the pool
  // (lo, hi) and its valid slot count
  __shared__ int4 s_stage[KVC_MAX_SPLIT_STAGES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);   // same value, known uniform
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  // Work-groups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of work items so one head's splits share an L2.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * p.items_per_xcd + (bid >> 3);
  if (item >= p.num_items) return;

  const int nstreams = p.plan[KVC_HDR_NUM_STREAMS];
  const kvc_dev_stream* recs = reinterpret_cast<const kvc_dev_stream*>(p.plan + KVC_PLAN_HEADER_INTS);
  int si = 0;
  while (si + 1 < nstreams && item >= recs[si + 1].item0) ++si;
  const kvc_dev_stream st = recs[si];
  const int32_t* kvidx = p.plan + KVC_PLAN_HEADER_INTS + KVC_STREAM_REC_INTS * nstreams + st.page0;

  int local = item - st.item0;
  const int grp = local % st.n_group;
  local /= st.n_group;
  const int split = local % st.n_split;
  const int h = local / st.n_split;

  const int nqt = (st.n_q + KVC_Q_TILE - 1) / KVC_Q_TILE;
  const int t_lo = grp * nqt / st.n_group;
  const int t_hi = (grp + 1) * nqt / st.n_group;
  const int ntile = t_hi - t_lo;
  const bool has_shared = ntile >= 5 && (ntile & 3) == 1;
  const int n_own = ntile - (has_shared ? 1 : 0);
  const int u0 = split * st.n_units / st.n_split;
  const int u1 = (split + 1) * st.n_units / st.n_split;
  const int nstage = u1 - u0;
  const float sl = p.scale_log2;
  const int H = p.num_heads;
  const uint32_t slot_bytes = (uint32_t)H * D * 2;

  // Stage table of this split.  Unit u is the 64-slot chunk cu of visible
  // page pi: patch pages hold P valid slots, special pages page_size, the
  // last page last_len ([p1] "How FlashInfer KV Cache Attention Accelerates
  // Streaming 3D Reconstruction Over SDPA" §Efficient Attention Masking and
  // Padding: lengths, not masks, delimit the valid tokens).
  for (int i = tid; i < nstage; i += 256) {
    const int u = u0 + i;
    const int patch_units = st.n_patch * st.upp;
    int pi, cu;
    if (u < patch_units) {
      pi = u / st.upp;
      cu = u - pi * st.upp;
    } else {
      const int pj = (u - patch_units) / st.ups;
      pi = st.n_patch + pj;
      cu = u - patch_units - pj * st.ups;
    }
    const int len = pi == st.n_pages - 1 ? st.last_len : (pi < st.n_patch ? p.patch_tokens : p.page_size);
    const uint64_t off = (((uint64_t)kvidx[pi] * 2) * p.page_size + (uint64_t)KT * cu) * slot_bytes +
                         (uint64_t)h * D * 2;
    s_stage[i] = int4{(int)(uint32_t)off, (int)(uint32_t)(off >> 32), min(KT, len - KT * cu), 0};
  }

  // ---- query operands (Q^T as the MFMA B operand) ----
  auto load_q = [&](int tile, bool ok, bf16x8 (&q)[S::KSTEPS]) {
    const int row = KVC_Q_TILE * tile + r16;
    ok = ok && row < st.n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)(st.q_row0 + (ok ? row : 0)) * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      q[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g4);
      if (!ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[ks][j] = (__bf16)0.0f;
      }
    }
  };
  int ntw = 0;
#pragma unroll
  for (int k = 0; k < QTW; ++k)
    if (wave + KVC_ATTN_WAVES * k < n_own) ntw = k + 1;

  bf16x8 qop[QTW][S::KSTEPS];
  float mb_run[QTW], l_run[QTW];
  f32x4 oacc[QTW][S::DBLK];
#pragma unroll
  for (int k = 0; k < QTW; ++k) {
    load_q(t_lo + wave + KVC_ATTN_WAVES * k, k < ntw, qop[k]);
    mb_run[k] = -INFINITY;
    l_run[k] = 0.0f;
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db) oacc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 qsh[S::KSTEPS];
  float mb_sh = -INFINITY, l_sh = 0.0f;
  f32x4 osh[S::DBLK];
  load_q(t_hi - 1, has_shared, qsh);
#pragma unroll
  for (int db = 0; db < S::DBLK; ++db) osh[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();   // stage table ready

  // ---- direct global -> LDS loads of one stage (K rows, then V rows) ----
  // Load instruction i of a stage fills 1 KiB of LDS, lane l writing bytes
  // [16 l, 16 l + 16); the lane fetches the logical chunk that the swizzle
  // places there, from the stage's uniform base address plus a per-lane
  // offset.  In a partial stage, rows past the valid count re-read the last
  // valid row (finite data; their scores are masked to -inf).
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  const uint64_t v_half = (uint64_t)p.page_size * slot_bytes;
  int lrow[S::LOADS_PER_WAVE];
  uint32_t lofs[S::LOADS_PER_WAVE];
#pragma unroll
  for (int j = 0; j < S::LOADS_PER_WAVE; ++j) {
    const int inst = wave * S::LOADS_PER_WAVE + j;
    const int blk = inst % (S::LOADS / 2);
    const int off = blk * 1024 + lane * 16;
    const int row = off / S::ROW_BYTES;
    const int pch = (off % S::ROW_BYTES) >> 4;
    lrow[j] = row;
    lofs[j] = (uint32_t)((pch ^ (swz(row) & (S::CPR - 1))) << 4);
  }
  auto issue = [&](int sidx) {
    const int4 e = s_stage[sidx];
    const uint64_t koff = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(e.x) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(e.y) << 32);
    const int valid = __builtin_amdgcn_readfirstlane(e.z);
    uint8_t* stage = ring + (sidx % S::NSTAGE) * S::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < S::LOADS_PER_WAVE; ++j) {
      const int inst = wave * S::LOADS_PER_WAVE + j;
      const int kv = inst >= S::LOADS / 2 ? 1 : 0;
      const int blk = inst - kv * (S::LOADS / 2);
      const uint32_t vofs = (uint32_t)min(lrow[j], valid - 1) * slot_bytes + lofs[j];
      const uint64_t b = (uint64_t)(uintptr_t)(pool + koff + (kv ? v_half : 0));
      const uint64_t ub = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
      load_lds16((const void*)(uintptr_t)ub, vofs,
                 __builtin_amdgcn_readfirstlane(lds_addr(stage + kv * S::HALF_BYTES + blk * 1024)));
    }
  };

  // ---- one stage of 64 slots for this wave's tiles ----
  auto compute = [&](int sidx, int valid) {
    const uint8_t* kb = ring + (sidx % S::NSTAGE) * S::STAGE_BYTES;
    const uint8_t* vb = kb + S::HALF_BYTES;
    // K operand rows: block kbi (= 2*pair + half) row r16 holds kv
    // 32*pair + 8*(r16/4) + 4*half + r16%4, so that after the MFMA lane group
    // g4 holds kv 32*pair + 8*g4 + [0, 8) of each query column.
    bf16x8 kop[4][S::KSTEPS];
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi) {
      const int kvrow = 32 * (kbi >> 1) + 8 * (r16 >> 2) + 4 * (kbi & 1) + (r16 & 3);
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks) {
        const int chunk = 4 * ks + g4;
        kop[kbi][ks] = *reinterpret_cast<const bf16x8*>(kb + kvrow * S::ROW_BYTES +
                                                        ((chunk ^ (swz(kvrow) & (S::CPR - 1))) << 4));
      }
    }
    // V^T operands by transposing reads of row-major V: lane (g4, r16) gets
    // V[32*pair + 8*g4 + j][16*db + r16], j = 0..7.
    bf16x8 vop[S::DBLK][2];
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        i16x4 half[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 32 * pp + 8 * g4 + 4 * r + (r16 >> 2);
          const int chunk = 2 * db + ((r16 & 3) >> 1);
          half[r] = ds_read_tr16(vb + row * S::ROW_BYTES + ((chunk ^ (swz(row) & (S::CPR - 1))) << 4) +
                                 ((r16 & 1) << 3));
        }
        const i16x4 a = half[0], b = half[1];
        vop[db][pp] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                                     a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
      }
    }
    // This wave's block of the shared tile (wave-uniform index).
    const bool sh_live = has_shared && (wv == 0   ? T::template block_live<0>(valid)
                                        : wv == 1 ? T::template block_live<1>(valid)
                                        : wv == 2 ? T::template block_live<2>(valid)
                                                  : T::template block_live<3>(valid));
    auto sh_qk = [&]() -> f32x4 {
      switch (wv) {
        case 0: return T::template shared_qk<0>(kop, qsh);
        case 1: return T::template shared_qk<1>(kop, qsh);
        case 2: return T::template shared_qk<2>(kop, qsh);
        default: return T::template shared_qk<3>(kop, qsh);
      }
    };
    // Own tiles, software-pipelined: the QK^T of the next tile (or of the
    // shared block, after the last own tile) is issued before the softmax of
    // the current one, so no MFMA result is read right after it is issued.
    f32x4 sacc[2][4];
    f32x4 ssh = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ntw > 0)
      T::qk(kop, qop[0], sacc[0]);
    else if (sh_live)
      ssh = sh_qk();
#pragma unroll
    for (int k = 0; k < QTW; ++k) {
      if (k < ntw) {
        if (k + 1 < ntw)
          T::qk(kop, qop[k + 1], sacc[(k + 1) & 1]);
        else if (sh_live)
          ssh = sh_qk();
        bf16x8 pb[2];
        T::softmax(sacc[k & 1], valid, g4, sl, mb_run[k], l_run[k], oacc[k], pb);
        T::pv(vop, pb, oacc[k]);
      }
    }
    if (sh_live) {
      switch (wv) {
        case 0: T::template shared_rest<0>(ssh, vop, valid, g4, sl, mb_sh, l_sh, osh); break;
        case 1: T::template shared_rest<1>(ssh, vop, valid, g4, sl, mb_sh, l_sh, osh); break;
        case 2: T::template shared_rest<2>(ssh, vop, valid, g4, sl, mb_sh, l_sh, osh); break;
        default: T::template shared_rest<3>(ssh, vop, valid, g4, sl, mb_sh, l_sh, osh); break;
      }
    }
  };

#pragma unroll
  for (int d = 0; d < S::DIST; ++d)
    if (d < nstage) issue(d);
  for (int sidx = 0; sidx < nstage; ++sidx) {
    if (sidx + S::DIST < nstage) issue(sidx + S::DIST);
    const int ahead = min(S::DIST, nstage - 1 - sidx);
    if (ahead >= 2)
      wait_vmcnt<2 * S::LOADS_PER_WAVE>();
    else if (ahead == 1)
      wait_vmcnt<S::LOADS_PER_WAVE>();
    else
      wait_vmcnt<0>();
    block_barrier();
    compute(sidx, __builtin_amdgcn_readfirstlane(s_stage[sidx].z));
  }

  // The epilogue reads the accumulators the last stage's MFMAs wrote; give
  // those MFMAs their result latency regardless of how the loop exit is laid
  // out (the compiler's wait states were not always inserted across branches).
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

  // ---- epilogue ----
  auto store = [&](int tile, float mb, float l, const f32x4 (&o)[S::DBLK]) {
    const float inv = 1.0f / l;
    const int row = KVC_Q_TILE * tile + r16;
    if (row >= st.n_q) return;
    const int grow = st.q_row0 + row;
    if (st.n_split == 1) {
      uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)grow * H + h) * D;
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) {
        const f32x4 v = o[db] * inv;
        bf16x4 b;
        b[0] = (__bf16)v[0];
        b[1] = (__bf16)v[1];
        b[2] = (__bf16)v[2];
        b[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * g4) = b;
      }
    } else {
      const size_t prow = ((size_t)split * p.rows_cap + grow) * H + h;
      float* po = p.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) *reinterpret_cast<f32x4*>(po + 16 * db + 4 * g4) = o[db] * inv;
      if (g4 == 0) p.part_lse[prow] = mb + __log2f(l);
    }
  };
#pragma unroll
  for (int k = 0; k < QTW; ++k)
    if (k < ntw) store(t_lo + wave + KVC_ATTN_WAVES * k, mb_run[k], lane_swap_sum(l_run[k]), oacc[k]);

  if (has_shared) {
    // merge the four waves' partial states of the shared tile (one split
    // merge: weights 2^(m_w - max m))
    constexpr int NV = S::DBLK * 4 + 2;
    float* xs = reinterpret_cast<float*>(ring);
    const float lt = lane_swap_sum(l_sh);
    __syncthreads();   // every wave is done with the ring
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[(wave * 64 + lane) * NV + 4 * db + i] = osh[db][i];
    xs[(wave * 64 + lane) * NV + S::DBLK * 4] = mb_sh;
    xs[(wave * 64 + lane) * NV + S::DBLK * 4 + 1] = lt;
    __syncthreads();
    if (wave == 0) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < KVC_ATTN_WAVES; ++w) M = fmaxf(M, xs[(w * 64 + lane) * NV + S::DBLK * 4]);
      float lsum = 0.f;
      f32x4 o[S::DBLK];
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < KVC_ATTN_WAVES; ++w) {
        const float* x = xs + (w * 64 + lane) * NV;
        const float wt = __builtin_amdgcn_exp2f(x[S::DBLK * 4] - M);
        lsum += wt * x[S::DBLK * 4 + 1];
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[db][i] += wt * x[4 * db + i];
      }
      store(t_hi - 1, M, lsum, o);
    }
  }
}

// ---------------------------------------------------------------------------
// merge of KV splits
// ---------------------------------------------------------------------------
// One wave per (row, head): lanes are split into groups of D/4 lanes (four
// floats each); group g accumulates splits g, g + groups, ... weighted by
// 2^(lse_c - max lse), and the groups are summed by lane exchanges.  The
// order of every sum is fixed, so the result does not depend on timing.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int LPR = D / 4;   // lanes per output row
  constexpr int SG = 64 / LPR; // split groups per wave
  const int lane = threadIdx.x & 63;
  const int gid = blockIdx.x * 4 + ((int)threadIdx.x >> 6);
  const int H = p.num_heads;
  const int row = gid / H;
  const int h = gid - row * H;
  if (row >= p.num_rows) return;
  const int nstreams = p.plan[KVC_HDR_NUM_STREAMS];
  const kvc_dev_stream* recs = reinterpret_cast<const kvc_dev_stream*>(p.plan + KVC_PLAN_HEADER_INTS);
  int si = 0;
  while (si + 1 < nstreams && row >= recs[si + 1].q_row0) ++si;
  const int nsp = recs[si].n_split;
  if (nsp <= 1) return;
  const size_t stride = (size_t)p.rows_cap * H;
  const size_t base = (size_t)row * H + h;
  float m = -INFINITY;
  for (int c = lane; c < nsp; c += 64) m = fmaxf(m, p.part_lse[c * stride + base]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const int sg = lane / LPR, lr = lane % LPR;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll 4
  for (int c = sg; c < nsp; c += SG) {
    const size_t prow = c * stride + base;
    const float w = __builtin_amdgcn_exp2f(p.part_lse[prow] - m);
    acc += w * *reinterpret_cast<const f32x4*>(p.part_o + prow * D + 4 * lr);
    wsum += w;
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
    wsum += __shfl_xor(wsum, off);
  }
  if (sg != 0) return;
  const f32x4 v = acc * (1.0f / wsum);
  bf16x4 b;
  b[0] = (__bf16)v[0];
  b[1] = (__bf16)v[1];
  b[2] = (__bf16)v[2];
  b[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + base * D + 4 * lr) = b;
}

}  // namespace

int launch_append(const AppendParams& p, void* s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.T), dim3(256), 0, (hipStream_t)s, p);
  return (int)hipGetLastError();
}

int launch_attention(const AttnParams& p, int32_t grid, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  switch (p.head_dim) {
    case 32:
      hipLaunchKernelGGL((attn_kernel<32, KVC_QTW_SMALL_D>), dim3(grid), dim3(256), 0, hs, p);
      break;
    case 64:
      hipLaunchKernelGGL((attn_kernel<64, KVC_QTW_SMALL_D>), dim3(grid), dim3(256), 0, hs, p);
      break;
    case 128:
      hipLaunchKernelGGL((attn_kernel<128, 4>), dim3(grid), dim3(256), 0, hs, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_merge(const MergeParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  const int grid = (p.num_rows * p.num_heads + 3) / 4;   // one wave per (row, head)
  switch (p.head_dim) {
    case 32:
      hipLaunchKernelGGL(merge_kernel<32>, dim3(grid), dim3(256), 0, hs, p);
      break;
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, hs, p);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, hs, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace kvc
