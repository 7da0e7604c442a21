// Host page allocator and per-step planner of the two-stream paged KV cache.
// Plain C++17: no HIP headers, so it builds and is tested with the host
// compiler alone.
//
// Page bookkeeping follows [p1] "How FlashInfer KV Cache Attention Accelerates
// Streaming 3D Reconstruction Over SDPA" §Two-Stream Design for Token Types
// (deques of free / scale / live-window patch pages; append-only special
// pages) and [p3] "How FlashInfer's Paged KV Cache Attention Outperforms SDPA
// Fallback in Streaming Inference" §Two-Stream Design (one patch page per
// frame; specials pack continuously across pages).
#ifndef KVC_HOST_HPP
#define KVC_HOST_HPP

#include <cstdint>
#include <deque>
#include <string>
#include <vector>

#include "kvc_plan_layout.h"

namespace kvc {

struct Config {
  int32_t num_blocks = 0, num_heads = 0, head_dim = 0, tokens_per_frame = 0;
  int32_t num_special_tokens = 0, special_row_offset = 0, page_size = 0;
  int32_t scale_frames = 0, sliding_window = 0, num_streams = 0;
  int32_t max_patch_pages = 0, max_special_pages = 0;
  int32_t max_frames_per_step = 1;
  int32_t dtype = 0;   // element type: 0 bfloat16, 1 float16, 2 float32

  int32_t patch_tokens() const { return tokens_per_frame - num_special_tokens; }
  int32_t max_num_pages() const { return max_patch_pages + max_special_pages; }
  int32_t rows_capacity() const { return num_streams * max_frames_per_step * tokens_per_frame; }
  // query tiles of KVC_Q_TILE32 rows over all streams (split partial outputs)
  int32_t tiles_capacity() const {
    return num_streams * ((max_frames_per_step * tokens_per_frame + KVC_Q_TILE32 - 1) / KVC_Q_TILE32);
  }
  int32_t elem_bytes() const { return dtype == 2 ? 4 : 2; }
  // float32 pools have an attention kernel of their own (one wave per 16
  // query rows, no split)
  bool fp32() const { return dtype == 2; }
  // of the 16-bit kernels, the 32x32 one serves head_dim 32 and 64, the
  // 16x16 one 128
  bool tiles32() const { return head_dim <= 64 && !fp32(); }
};

// Result codes mirror kvc_status.
enum Code { OK = 0, ERR_ARG = -1, ERR_STATE = -2, ERR_POOL = -3, ERR_CAPACITY = -4, ERR_UNSUPPORTED = -6 };

// Validates a configuration; returns OK or an error code with a message.
int validate(const Config& c, std::string* why);

// Where one frame's tokens go.  Special token j of the frame is at page
// sp_pages[(sp_slot0 + j) / page_size], slot (sp_slot0 + j) % page_size.
struct FrameSlots {
  int32_t patch_page = -1;
  int32_t sp_slot0 = 0;
  int32_t n_sp_pages = 0;
  int32_t sp_pages[KVC_MAX_APPEND_SPECIAL_PAGES] = {0};
};

struct StreamState {
  std::vector<int32_t> scale_pages;    // permanent, in frame order
  std::deque<int32_t> live_pages;      // sliding window, oldest first
  std::vector<int32_t> special_pages;  // append-only
  int64_t special_tokens = 0;
  int64_t frame_count = 0;
  // deferred eviction: window pages evicted since the last frame's append,
  // oldest first; out of the visible table but not yet free
  std::vector<int32_t> pending;
  bool last_is_live = false;   // the last frame's patch page went to the window
  bool can_rollback = false;   // the last frame may still be undone
};

class Allocator {
 public:
  // free_patch_order / free_special_order may be empty (ascending IDs).
  int init(const Config& cfg, const std::vector<int32_t>& free_patch_order,
           const std::vector<int32_t>& free_special_order, std::string* why);
  void reset();
  // Allocate one frame of `stream`; state is unchanged on error.  With
  // deferred eviction, pages held back by the previous evict are released to
  // the free list first (the previous frame can no longer be undone).
  int append(int stream, FrameSlots* out, std::string* why);
  // Undo the stream's most recent frame (deferred eviction only): its patch
  // page and the special pages it opened go back to the front of the free
  // lists, its special tokens are dropped, and held-back window pages return
  // to the front of the window until it is full again.  ERR_STATE when there
  // is nothing to undo.
  int rollback(int stream, std::string* why);
  void set_defer_eviction(bool on) { defer_ = on; }
  bool defer_eviction() const { return defer_; }
  // Free live-window pages beyond the window; returns the number freed.
  int evict(int stream);

  const Config& config() const { return cfg_; }
  const StreamState& stream(int s) const { return streams_[s]; }
  int32_t free_patch_count() const { return (int32_t)free_patch_.size(); }
  int32_t free_special_count() const { return (int32_t)free_special_.size(); }
  // Valid tokens on the last page of the stream's visible table ([p5] "How
  // Paged KV Cache Attention Achieves Stable Inference in Ling-Bot-Map"
  // §Kernel Dispatch and Sequence Lengths).
  int32_t last_page_len(int stream) const;

 private:
  Config cfg_;
  std::vector<int32_t> init_patch_, init_special_;
  std::deque<int32_t> free_patch_, free_special_;
  std::vector<StreamState> streams_;
  bool defer_ = false;
};

// Split / group policy of the attention launch.
struct PlanPolicy {
  int32_t target_workgroups = 512;
  int32_t max_splits = KVC_MAX_SPLITS;
  // head_dim 64, 16-bit pools: 0 = the kernel whose launch the cost model
  // finds shorter, 16 / 32 = the 16x16 / 32x32 kernel always
  int32_t query_tile = 0;
  // Fused append: the work units of the step's own frames are cut where
  // their input rows stop being consecutive (so that a unit can be read
  // from the caller's k / v rows instead of the pool), and the plan carries
  // the pool row of every input row (the copy that the merge launch makes).
  bool fused = false;
};

// Host image of one step's plan.
struct HostPlan {
  std::vector<int32_t> planned;        // stream ids, ascending
  std::vector<int32_t> kv_indptr;      // size n+1
  std::vector<int32_t> kv_indices;
  std::vector<int32_t> last_page_len;
  std::vector<int32_t> n_patch_pages;
  std::vector<int32_t> qo_indptr;      // size n+1
  std::vector<int32_t> n_split;
  std::vector<int32_t> image;          // device layout (kvc_plan_layout.h)
  int32_t num_items = 0;
  int32_t num_rows = 0;
  int32_t num_tiles = 0;
  bool shared_tile = true;             // launch variant (KVC_HDR_SHARED_TILE): 32x32 kernel: groups may carry a
                                       // 16-row tail; 16x16 kernel: groups with a shared ninth tile
  bool tiles16 = false;                // head_dim 64 served by the 16x16 kernel (KVC_VARIANT_TILES16)
  int32_t merge_table = 0;             // offset in ints of the merge order in image
  int32_t merge_slots = 0;             // merge slots per XCD
  bool any_split = false;
  bool fused = false;                  // built with PlanPolicy::fused
  int32_t copy_table = 0;              // fused: offset in ints of the input rows' pool rows
};

// Plan the given streams (ascending) from the allocator's current lists.
// frames[i]: frames streams[i] appended this step (its queries are
// frames[i] * tokens_per_frame rows).  slots[i]: the placement of those
// frames (read only with PlanPolicy::fused).
void build_plan(const Allocator& a, const std::vector<int32_t>& streams, const std::vector<int32_t>& frames,
                const std::vector<const FrameSlots*>& slots, const PlanPolicy& pol, HostPlan* out);

// Pool row (the K row; V is page_size rows further) that input row t of
// frame fs takes: the frame's patch page for patch rows, its special slots
// for the special rows [special_row_offset, + num_special_tokens).
uint32_t input_row_slot(const Config& c, const FrameSlots& fs, int32_t t);

// int32 entries of the device plan image for a configuration (upper bound).
size_t plan_image_ints(const Config& c);

}  // namespace kvc

#endif
