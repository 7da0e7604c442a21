// Launch interface of the HIP kernels (plain types; no HIP headers needed).
#ifndef KVC_KERNELS_H
#define KVC_KERNELS_H

#include <stddef.h>
#include <stdint.h>

#include "kvc_plan_layout.h"

namespace kvc {

struct AppendParams {
  void* pool;               // this block's pool
  const void* k;            // [T, H, D] of the element type
  const void* v;
  int32_t T, row_elems;     // row_elems = H * D
  int32_t elem_bytes;       // 2 (bf16, f16) or 4 (float32)
  int32_t special_row_offset, n_special, page_size;
  int32_t patch_page, sp_slot0, n_sp_pages;
  int32_t sp_pages[KVC_MAX_APPEND_SPECIAL_PAGES];
  // rotary embedding of K: float32 [T, D/2] cos and sin of this frame's
  // rows, 16-byte aligned, or both null to store K as it is
  const float* rope_cos;
  const float* rope_sin;
  int32_t head_dim;
  int32_t dtype;            // element type: 0 bfloat16, 1 float16, 2 float32
};

struct RopeParams {
  const void* x;            // [rows, H, D] elements of the element type
  void* y;                  // same shape, written; must not overlap x
  const float* cos;         // [rows, D/2] float32, 16-byte aligned
  const float* sin;
  int64_t chunks;           // 16-byte chunks: rows * H * D * elem bytes / 16
  int32_t row_elems, head_dim;
  int32_t dtype;
};

struct AttnParams {
  const int32_t* plan;      // device plan image
  const void* pool;
  const void* q;            // [R, H, D] bf16
  void* o;                  // [R, H, D] bf16
  // Split partial outputs, per query tile of 32 rows, in the lane order of the
  // 32x32 MFMA accumulators so that each store instruction of that kernel
  // writes 512 contiguous bytes: part_o[split][head][tile][d / 32][(d % 32) / 8]
  // [lane][4] bf16 (normalised; lane = 32 * ((d % 8) / 4) + row % 32, the last
  // index d % 4), part_lse[split][head][tile][32] float (base-2 log-sum-exp).
  void* part_o;
  float* part_lse;
  int32_t num_heads, head_dim, page_size, patch_tokens, tiles_cap;   // tiles_cap: 32-row tiles
  float scale_log2;         // log2(e) / sqrt(D)
  int32_t num_items, items_per_xcd;
  int32_t shared_tile;      // launch variant, as KVC_HDR_SHARED_TILE of the plan
  int32_t dtype;            // element type: 0 bfloat16, 1 float16
  // The plan's stream count and, when it is at most KVC_ARG_STREAMS, copies
  // of its stream records (the 32x32 kernel then starts its unit-entry loads
  // without first loading the plan's header and records)
  int32_t num_streams;
  kvc_dev_stream recs[KVC_ARG_STREAMS];
  // Fused append (32x32 kernel, at most KVC_ARG_STREAMS streams): 1 when the
  // units of the step's own rows are read from kin / vin (per stream, in
  // plan order: the frames' rows in query order) instead of the pool
  int32_t fused;
  const void* kin[KVC_ARG_STREAMS];
  const void* vin[KVC_ARG_STREAMS];
};

struct MergeParams {
  const int32_t* plan;
  const void* part_o;       // bf16
  const float* part_lse;
  void* o;
  int32_t num_heads, head_dim, tiles_cap, num_tiles;
  int32_t max_split;        // largest split count over the planned streams
  int32_t merge_table;      // offset in ints of the plan's merge order
  int32_t merge_slots;      // merge slots per XCD
  int32_t dtype;            // element type: 0 bfloat16, 1 float16
  // Fused append: after the KVC_NUM_XCD * merge_slots merge work-groups,
  // copy_wgs work-groups copy the step's input rows (copy_rows of them, the
  // streams' own frames in query order, stream i's from row row0[i]) into
  // the pool, at the K rows the plan's copy table gives (V page_size rows
  // further); row_bytes = H * D * element size
  int32_t copy_wgs, copy_rows, copy_table, page_size, row_bytes, num_streams;
  int32_t row0[KVC_ARG_STREAMS + 1];
  void* pool;
  const void* kin[KVC_ARG_STREAMS];
  const void* vin[KVC_ARG_STREAMS];
};

// Copies per thread of the merge launch's copy work-groups (fused append).
#define KVC_COPY_PER 4

// Return 0 on success or the hipError_t value.
int launch_append(const AppendParams& p, void* hip_stream);
int launch_rope(const RopeParams& p, void* hip_stream);
int launch_attention(const AttnParams& p, int32_t grid, void* hip_stream);     // 16x16 kernel, head_dim 128
int launch_attention32(const AttnParams& p, int32_t grid, void* hip_stream);   // 32x32 kernel, head_dim 32, 64
int launch_attention_f32(const AttnParams& p, void* hip_stream);               // float32 pools, every head_dim
int launch_merge(const MergeParams& p, void* hip_stream);
// Device address and size of the static scratch of kvc_run_no_alloc on the
// current device (looked up once per device); 0 or the hipError_t value.
int no_alloc_scratch(void** ptr, size_t* bytes);

}  // namespace kvc

#endif
