// Device-side plan layout: what kvc_plan uploads once per frame step and every
// kvc_run of that step reads ([p3] "How FlashInfer's Paged KV Cache Attention
// Outperforms SDPA Fallback in Streaming Inference", §Plan-Run Execution
// Workflow: plan once at block 0, reuse in every block).
//
// Plain C layout, included by the host planner and by the HIP kernels.
//
// Buffer of int32:
//   [0, KVC_PLAN_HEADER_INTS)                      header
//   [.., + KVC_STREAM_REC_INTS * num_streams)      one record per planned stream
//   [.., + total visible pages)                    kv_indices: concatenated page
//                                                  tables, scale -> live -> special
//   [aligned to 4 ints, + 4 * total units)         unit tables: per stream, per
//                                                  64-slot work unit in table order,
//                                                  {slot index of its first K row, valid slots, 0, 0}
//   [aligned to 4 ints, + 4 * 8 * merge slots)     merge order: for each of the 8
//                                                  XCDs, the (query tile, head)
//                                                  pairs of split streams to merge
//                                                  there, {tile * H + head, KV
//                                                  splits, first output row, valid
//                                                  rows}, padded with pair -1
#ifndef KVC_PLAN_LAYOUT_H
#define KVC_PLAN_LAYOUT_H

#include <stdint.h>

#define KVC_PLAN_HEADER_INTS 8
#define KVC_STREAM_REC_INTS 20

// Slots per attention pipeline stage.  A stage never straddles a page: the
// work unit is (page, 64-slot chunk of that page's valid slots), so a stage
// is one contiguous run of slots.  Splits are ranges of units.
#define KVC_KV_TILE 64
// Query rows per MFMA tile, and waves per attention work-group, of the
// 16x16 attention kernel (head_dim 128).
#define KVC_Q_TILE 16
#define KVC_ATTN_WAVES 4
// The 32x32 attention kernel (head_dim 32 and 64): query groups of 8 tiles
// of 32 rows, one per wave of an 8-wave work-group, and a tail tile of up to
// 16 rows shared by the first 4 waves.  Split partial outputs of both
// kernels are stored per 32-row tile.
#define KVC_Q_TILE32 32
#define KVC_ATTN32_WAVES 8
#define KVC_GROUP_TILES32 8
#define KVC_TAIL_WAVES 4
#define KVC_TAIL_ROWS 16
// Query rows per work item (one wave) of the float32 attention kernel.
#define KVC_F32_ROWS 16
// Upper bound of KV splits per stream (sizes the partial-output workspace).
#define KVC_MAX_SPLITS 64
// Ints per work-unit entry: slot index of the unit's first K row in the
// block's pool [pages][2][page_size] (a uint32; times H * D * 2 bytes), its
// valid slot count, padding.
#define KVC_UNIT_INTS 4
// Most units (stages) one split of the 32x32 kernel covers: it keeps its
// split's unit entries in registers, 64 per register.
#define KVC_MAX_SPLIT_STAGES 512
// Largest n_s, and the most special pages one frame's specials can touch.
#define KVC_MAX_SPECIAL_PER_FRAME 64
#define KVC_MAX_APPEND_SPECIAL_PAGES 8

// Header fields.
#define KVC_HDR_NUM_STREAMS 0
#define KVC_HDR_NUM_ITEMS 1
#define KVC_HDR_NUM_ROWS 2
#define KVC_HDR_ANY_SPLIT 3
#define KVC_HDR_NUM_TILES 4
#define KVC_HDR_SHARED_TILE 5  // launch variant: bit 0: 32x32 kernel: query groups may carry a shared
                               // 16-row tail; 16x16 kernel: groups of up to 9 tiles (a shared ninth)
                               // instead of 8; bit 1 (KVC_VARIANT_TILES16): head_dim 64 served by the
                               // 16x16 kernel
#define KVC_VARIANT_TILES16 2
#define KVC_HDR_MERGE_TABLE 6  // offset in ints of the merge order
#define KVC_HDR_MERGE_SLOTS 7  // merge slots per XCD (the merge grid is 8 times this)
// XCDs of the device; work-groups are dispatched to them round-robin.
#define KVC_NUM_XCD 8
// Ints per merge-order entry.
#define KVC_MERGE_INTS 4

typedef struct kvc_dev_stream {
  int32_t q_row0;     // first query/output row of this stream
  int32_t n_q;        // query rows (T)
  int32_t page0;      // offset of this stream's table in kv_indices
  int32_t n_patch;    // patch pages in the table (scale + live)
  int32_t n_pages;    // pages in the table
  int32_t last_len;   // valid tokens on the last page
  int32_t kv_len;     // valid visible tokens L
  int32_t unit0;      // offset in ints of this stream's unit table from the plan start
  int32_t n_units;    // work units (64-slot chunks of the visible pages; fused plans cut the own frames' further)
  int32_t n_split;    // KV splits
  int32_t n_group;    // query groups (work-groups per head and split)
  int32_t item0;      // first attention work item of this stream
  int32_t n_items;    // H * n_split * n_group
  int32_t upp;        // units per patch page, ceil(P / KVC_KV_TILE)
  int32_t ups;        // units per full special page, ceil(page_size / KVC_KV_TILE)
  int32_t q_tile0;    // first 32-row query tile of this stream in the split partial outputs
  int32_t n_t32;      // 32x32 kernel: full 32-row query tiles shared out over the groups
  int32_t tail;       // 32x32 kernel: 1 if rows [32 n_t32, n_q) (at most 16) form the last group's tail
  int32_t reserved0, reserved1;
} kvc_dev_stream;

// Stream records the attention launch also passes by value.
#define KVC_ARG_STREAMS 4

// Query tiles (of KVC_Q_TILE rows) one wave owns.  A query group spans at
// most KVC_ATTN_WAVES * this many tiles, plus one tile shared by all waves
// when the launch uses shared tiles.
#define KVC_TILES_PER_WAVE 2
static inline int kvc_group_tiles(int shared_tile) {
  return KVC_ATTN_WAVES * KVC_TILES_PER_WAVE + (shared_tile ? 1 : 0);
}

#endif
