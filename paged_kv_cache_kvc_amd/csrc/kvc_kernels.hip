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
// of 4 waves streams its split's KV tokens through LDS in stages of 64
// tokens, double-buffered: K row-major, V transposed (V^T[d][kv]) so that the
// P.V contraction over kv reads 8 consecutive kv per lane.  The scores are
// computed transposed, S^T = K Q^T (16x16x32 bf16 MFMA, kv on rows, queries on
// columns), so each lane's accumulators belong to one query column: the
// softmax column max needs only two cross-lane steps, and the probabilities
// feed the P.V MFMA (O^T = V^T P^T) straight from registers.  Each wave owns a
// set of 16-query tiles.
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
  static constexpr int KSTEPS = D / 32;                  // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 16;                    // 16-row blocks of O^T
  static constexpr int K_BYTES = KT * D * 2;             // K stage, row-major [kv][d]
  static constexpr int V_BYTES = D * KT * 2;             // V stage, transposed [d][kv]
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  // Loads: threads [0,128) bring K rows, [128,256) bring V as 4-token x
  // 8-dim blocks that they transpose in registers.
  static constexpr int K_PER_THREAD = KT * CPR / 128;
  static constexpr int K_ROWS_PER_PASS = 128 / CPR;
  static constexpr int V_BLOCKS = (KT / 4) * CPR;
  static constexpr int V_PER_THREAD = (V_BLOCKS + 127) / 128;
  static constexpr int STG = (K_PER_THREAD > 4 * V_PER_THREAD) ? K_PER_THREAD : 4 * V_PER_THREAD;
};

// LDS chunk swizzles (XOR on the 16-byte chunk index inside a row) that keep
// the MFMA operand reads and the transposing V writes spread over banks.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int d) { return (d ^ (d >> 3)) & 7; }

template <int D>
__device__ __forceinline__ const uint16_t* kv_row(const AttnParams& p, const kvc_dev_stream& st,
                                                  const int32_t* kvidx, int tok, int kv, int h) {
  int pi, slot;
  if (tok < st.patch_tok) {
    pi = (int)fdiv((uint32_t)tok, p.div_patch);
    slot = tok - pi * p.patch_tokens;
  } else {
    const int t2 = tok - st.patch_tok;
    const int pj = (int)fdiv((uint32_t)t2, p.div_page);
    pi = st.n_patch + pj;
    slot = t2 - pj * p.page_size;
  }
  const int page = kvidx[pi];
  return static_cast<const uint16_t*>(p.pool) +
         ((((size_t)page * 2 + kv) * p.page_size + slot) * p.num_heads + h) * D;
}

template <int D, int QTW>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int u0 = split * st.n_units / st.n_split;
  const int u1 = (split + 1) * st.n_units / st.n_split;
  const int tok0 = u0 * KT;
  const int tok1 = min(st.kv_len, u1 * KT);
  const int nstage = u1 - u0;
  const float sl = p.scale_log2;
  const int H = p.num_heads;

  // ---- this wave's query tiles: t_lo + wave + 4k ----
  int ntw = 0;
#pragma unroll
  for (int k = 0; k < QTW; ++k)
    if (t_lo + wave + KVC_ATTN_WAVES * k < t_hi) ntw = k + 1;

  bf16x8 qop[QTW][S::KSTEPS];
  float m_run[QTW], l_run[QTW];
  f32x4 oacc[QTW][S::DBLK];
#pragma unroll
  for (int k = 0; k < QTW; ++k) {
    const int row = KVC_Q_TILE * (t_lo + wave + KVC_ATTN_WAVES * k) + r16;
    const bool ok = k < ntw && row < st.n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)(st.q_row0 + row) * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      if (ok) {
        qop[k][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g4);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qop[k][ks][j] = (__bf16)0.0f;
      }
    }
    m_run[k] = -INFINITY;
    l_run[k] = 0.0f;
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db) oacc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- global -> registers -> LDS staging ----
  u32x4 stg[S::STG];
  auto load_stage = [&](int sidx) {
    const int base = tok0 + sidx * KT;
    const int valid = min(KT, tok1 - base);
    if (tid < 128) {
      const int cc = tid % S::CPR;
      const int rg = tid / S::CPR;
#pragma unroll
      for (int i = 0; i < S::K_PER_THREAD; ++i) {
        const int row = rg + S::K_ROWS_PER_PASS * i;
        if (row < valid)
          stg[i] = *reinterpret_cast<const u32x4*>(kv_row<D>(p, st, kvidx, base + row, 0, h) + cc * 8);
        else
          stg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const int u = tid - 128;
#pragma unroll
      for (int j = 0; j < S::V_PER_THREAD; ++j) {
        const int b = u + 128 * j;
        const int cc = b % S::CPR;
        const int kg = b / S::CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * kg + i;
          if (b < S::V_BLOCKS && row < valid)
            stg[4 * j + i] = *reinterpret_cast<const u32x4*>(kv_row<D>(p, st, kvidx, base + row, 1, h) + cc * 8);
          else
            stg[4 * j + i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* kb = smem + buf * S::STAGE_BYTES;
    uint8_t* vb = kb + S::K_BYTES;
    if (tid < 128) {
      const int cc = tid % S::CPR;
      const int rg = tid / S::CPR;
#pragma unroll
      for (int i = 0; i < S::K_PER_THREAD; ++i) {
        const int row = rg + S::K_ROWS_PER_PASS * i;
        *reinterpret_cast<u32x4*>(kb + row * (D * 2) + ((cc ^ (swz_k(row) & (S::CPR - 1))) << 4)) = stg[i];
      }
    } else {
      const int u = tid - 128;
#pragma unroll
      for (int j = 0; j < S::V_PER_THREAD; ++j) {
        const int b = u + 128 * j;
        if (b >= S::V_BLOCKS) continue;
        const int cc = b % S::CPR;
        const int kg = b / S::CPR;
        const u32x4 r0 = stg[4 * j + 0], r1 = stg[4 * j + 1], r2 = stg[4 * j + 2], r3 = stg[4 * j + 3];
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int w = dd >> 1;
          uint32_t lo, hi;
          if (dd & 1) {
            lo = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
            hi = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
          } else {
            lo = (r0[w] & 0xffffu) | (r1[w] << 16);
            hi = (r2[w] & 0xffffu) | (r3[w] << 16);
          }
          const int d = 8 * cc + dd;
          const int off = d * (KT * 2) + (((kg >> 1) ^ swz_v(d)) << 4) + ((kg & 1) << 3);
          *reinterpret_cast<u32x2*>(vb + off) = u32x2{lo, hi};
        }
      }
    }
  };

  auto compute_stage = [&](int buf, int valid) {
    const uint8_t* kb = smem + buf * S::STAGE_BYTES;
    const uint8_t* vb = kb + S::K_BYTES;
    // K operand rows: block kb_i (= 2*pair + half) row r16 holds kv
    // 32*pair + 8*(r16/4) + 4*half + r16%4, so that after the MFMA lane group
    // g4 holds kv 32*pair + 8*g4 + [0, 8) of each query column.
    bf16x8 kop[4][S::KSTEPS];
#pragma unroll
    for (int kbi = 0; kbi < 4; ++kbi) {
      const int kvrow = 32 * (kbi >> 1) + 8 * (r16 >> 2) + 4 * (kbi & 1) + (r16 & 3);
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks) {
        const int chunk = 4 * ks + g4;
        kop[kbi][ks] = *reinterpret_cast<const bf16x8*>(
            kb + kvrow * (D * 2) + ((chunk ^ (swz_k(kvrow) & (S::CPR - 1))) << 4));
      }
    }
    bf16x8 vop[S::DBLK][2];
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db) {
      const int d = 16 * db + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int chunk = 4 * pp + g4;
        vop[db][pp] = *reinterpret_cast<const bf16x8*>(vb + d * (KT * 2) + ((chunk ^ swz_v(d)) << 4));
      }
    }
#pragma unroll
    for (int k = 0; k < QTW; ++k) {
      if (k < ntw) {
        f32x4 sacc[4];
#pragma unroll
        for (int kbi = 0; kbi < 4; ++kbi) {
          sacc[kbi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < S::KSTEPS; ++ks)
            sacc[kbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kbi][ks], qop[k][ks], sacc[kbi], 0, 0, 0);
        }
        if (valid < KT) {
#pragma unroll
          for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (32 * (kbi >> 1) + 8 * g4 + 4 * (kbi & 1) + i >= valid) sacc[kbi][i] = -INFINITY;
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kbi][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[k], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[k] - m_new) * sl);
        m_run[k] = m_new;
        const float mb = m_new * sl;
        float lsum = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int kbi = 0; kbi < 4; ++kbi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbi][i], sl, -mb));
            lsum += pv;
            pb[kbi >> 1][4 * (kbi & 1) + i] = (__bf16)pv;
          }
        l_run[k] = l_run[k] * alpha + lsum;
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db) {
          oacc[k][db] *= alpha;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
            oacc[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db][pp], pb[pp], oacc[k][db], 0, 0, 0);
        }
      }
    }
  };

  if (nstage > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int sidx = 0; sidx < nstage; ++sidx) {
    const int buf = sidx & 1;
    const bool more = sidx + 1 < nstage;
    if (more) load_stage(sidx + 1);
    compute_stage(buf, min(KT, tok1 - (tok0 + sidx * KT)));
    if (more) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int k = 0; k < QTW; ++k) {
    if (k < ntw) {
      float l = l_run[k];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const float inv = 1.0f / l;
      const int row = KVC_Q_TILE * (t_lo + wave + KVC_ATTN_WAVES * k) + r16;
      if (row < st.n_q) {
        const int grow = st.q_row0 + row;
        if (st.n_split == 1) {
          uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)grow * H + h) * D;
#pragma unroll
          for (int db = 0; db < S::DBLK; ++db) {
            const f32x4 v = oacc[k][db] * inv;
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
          for (int db = 0; db < S::DBLK; ++db)
            *reinterpret_cast<f32x4*>(po + 16 * db + 4 * g4) = oacc[k][db] * inv;
          if (g4 == 0) p.part_lse[prow] = m_run[k] * sl + __log2f(l);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge of KV splits
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int LPR = D / 4;              // lanes per (row, head), 4 floats each
  constexpr int PER_BLOCK = 256 / LPR;
  const int gid = blockIdx.x * PER_BLOCK + (int)threadIdx.x / LPR;
  const int lr = (int)threadIdx.x % LPR;
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
  float M = -INFINITY;
  for (int c = 0; c < nsp; ++c) M = fmaxf(M, p.part_lse[((size_t)c * p.rows_cap + row) * H + h]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int c = 0; c < nsp; ++c) {
    const size_t prow = ((size_t)c * p.rows_cap + row) * H + h;
    const float w = __builtin_amdgcn_exp2f(p.part_lse[prow] - M);
    acc += w * *reinterpret_cast<const f32x4*>(p.part_o + prow * D + 4 * lr);
    wsum += w;
  }
  const f32x4 v = acc * (1.0f / wsum);
  bf16x4 b;
  b[0] = (__bf16)v[0];
  b[1] = (__bf16)v[1];
  b[2] = (__bf16)v[2];
  b[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + ((size_t)row * H + h) * D + 4 * lr) = b;
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
      hipLaunchKernelGGL((attn_kernel<32, 5>), dim3(grid), dim3(256), 0, hs, p);
      break;
    case 64:
      hipLaunchKernelGGL((attn_kernel<64, 5>), dim3(grid), dim3(256), 0, hs, p);
      break;
    case 128:
      hipLaunchKernelGGL((attn_kernel<128, 3>), dim3(grid), dim3(256), 0, hs, p);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_merge(const MergeParams& p, void* s) {
  const hipStream_t hs = (hipStream_t)s;
  const int per_block = 256 / (p.head_dim / 4);
  const int grid = (p.num_rows * p.num_heads + per_block - 1) / per_block;
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
