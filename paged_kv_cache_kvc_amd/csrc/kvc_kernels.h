// Launch interface of the HIP kernels (plain types; no HIP headers needed).
#ifndef KVC_KERNELS_H
#define KVC_KERNELS_H

#include <stddef.h>
#include <stdint.h>

#include "kvc_plan_layout.h"

namespace kvc {

struct AppendParams {
  void* pool;               // this block's pool
  const void* k;            // [T, H, D] bf16
  const void* v;
  int32_t T, row_elems;     // row_elems = H * D
  int32_t special_row_offset, n_special, page_size;
  int32_t patch_page, sp_slot0, n_sp_pages;
  int32_t sp_pages[KVC_MAX_APPEND_SPECIAL_PAGES];
};

struct AttnParams {
  const int32_t* plan;      // device plan image
  const void* pool;
  const void* q;            // [R, H, D] bf16
  void* o;                  // [R, H, D] bf16
  // Split partial outputs, per query tile of 16 rows, in the lane order of the
  // MFMA accumulators so that each store instruction writes 512 contiguous
  // bytes: part_o[split][head][tile][d block of 16][lane][4] bf16 (normalised;
  // lane = 16 * (d%16)/4 + row%16), part_lse[split][head][tile][16] float.
  void* part_o;
  float* part_lse;
  int32_t num_heads, head_dim, page_size, patch_tokens, tiles_cap;
  float scale_log2;         // log2(e) / sqrt(D)
  int32_t num_items, items_per_xcd;
  int32_t shared_tile;      // 1: query groups of up to 9 tiles, the ninth shared by the waves; 0: up to 8
  int32_t dtype;            // element type: 0 bfloat16, 1 float16
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
};

// Return 0 on success or the hipError_t value.
int launch_append(const AppendParams& p, void* hip_stream);
int launch_attention(const AttnParams& p, int32_t grid, void* hip_stream);
int launch_merge(const MergeParams& p, void* hip_stream);
// Device address and size of the static scratch of kvc_run_no_alloc on the
// current device (looked up once per device); 0 or the hipError_t value.
int no_alloc_scratch(void** ptr, size_t* bytes);

}  // namespace kvc

#endif
