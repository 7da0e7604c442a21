// Host page allocator and per-step planner (see kvc_host.hpp).
#include "kvc_host.hpp"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>

namespace kvc {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate(const Config& c, std::string* why) {
  auto fail = [&](int code, const char* msg) {
    if (why) *why = msg;
    return code;
  };
  if (c.num_blocks < 1 || c.num_heads < 1 || c.num_streams < 1) return fail(ERR_ARG, "num_blocks, num_heads and num_streams must be >= 1");
  if (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128) return fail(ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (c.tokens_per_frame < 1) return fail(ERR_ARG, "tokens_per_frame must be >= 1");
  if (c.num_special_tokens < 0 || c.num_special_tokens >= c.tokens_per_frame)
    return fail(ERR_ARG, "num_special_tokens must be in [0, tokens_per_frame)");
  if (c.num_special_tokens > KVC_MAX_SPECIAL_PER_FRAME) return fail(ERR_UNSUPPORTED, "num_special_tokens above 64");
  if (c.special_row_offset < 0 || c.special_row_offset + c.num_special_tokens > c.tokens_per_frame)
    return fail(ERR_ARG, "special rows [special_row_offset, +n_s) must lie inside the frame");
  if (c.page_size < c.patch_tokens() || c.page_size < 1) return fail(ERR_ARG, "page_size must be >= patch tokens");
  if (c.num_special_tokens > 0 &&
      ceil_div(c.page_size - 1 + c.num_special_tokens, c.page_size) > KVC_MAX_APPEND_SPECIAL_PAGES)
    return fail(ERR_UNSUPPORTED, "one frame's specials would span more than 8 special pages");
  if (c.scale_frames < 0 || c.sliding_window < 1) return fail(ERR_ARG, "scale_frames >= 0 and sliding_window >= 1 required");
  if (c.max_special_pages < 0 || c.max_patch_pages < 0) return fail(ERR_ARG, "page counts must be >= 0");
  if ((int64_t)c.max_patch_pages < (int64_t)c.num_streams * (c.scale_frames + c.sliding_window + 1))
    return fail(ERR_CAPACITY, "max_patch_pages must be >= num_streams * (scale_frames + sliding_window + 1)");
  const int64_t pages = (int64_t)c.max_patch_pages + c.max_special_pages;
  if (pages * c.page_size >= (int64_t)1 << 31) return fail(ERR_UNSUPPORTED, "pool slots per block must be < 2^31");
  if ((int64_t)c.num_heads * c.head_dim > 65536) return fail(ERR_UNSUPPORTED, "num_heads * head_dim above 65536");
  if (c.max_frames_per_step < 1 || c.max_frames_per_step > 64)
    return fail(ERR_ARG, "max_frames_per_step must be in [1, 64]");
  if (c.dtype < 0 || c.dtype > 2)
    return fail(ERR_UNSUPPORTED, "dtype must be KVC_DTYPE_BF16, KVC_DTYPE_F16 or KVC_DTYPE_F32");
  if ((int64_t)c.num_streams * c.max_frames_per_step * c.tokens_per_frame >= (int64_t)1 << 24)
    return fail(ERR_UNSUPPORTED, "too many query rows");
  return OK;
}

int Allocator::init(const Config& cfg, const std::vector<int32_t>& fp, const std::vector<int32_t>& fs,
                    std::string* why) {
  cfg_ = cfg;
  init_patch_.clear();
  init_special_.clear();
  if (fp.empty()) {
    for (int32_t i = 0; i < cfg.max_patch_pages; ++i) init_patch_.push_back(i);
  } else {
    if ((int32_t)fp.size() != cfg.max_patch_pages) {
      if (why) *why = "free_patch_order must list max_patch_pages IDs";
      return ERR_ARG;
    }
    std::vector<char> seen(cfg.max_patch_pages, 0);
    for (int32_t p : fp) {
      if (p < 0 || p >= cfg.max_patch_pages || seen[p]) {
        if (why) *why = "free_patch_order is not a permutation of [0, max_patch_pages)";
        return ERR_ARG;
      }
      seen[p] = 1;
    }
    init_patch_ = fp;
  }
  if (fs.empty()) {
    for (int32_t i = 0; i < cfg.max_special_pages; ++i) init_special_.push_back(cfg.max_patch_pages + i);
  } else {
    if ((int32_t)fs.size() != cfg.max_special_pages) {
      if (why) *why = "free_special_order must list max_special_pages IDs";
      return ERR_ARG;
    }
    std::vector<char> seen(cfg.max_special_pages, 0);
    for (int32_t p : fs) {
      const int32_t i = p - cfg.max_patch_pages;
      if (i < 0 || i >= cfg.max_special_pages || seen[i]) {
        if (why) *why = "free_special_order is not a permutation of [max_patch_pages, max_num_pages)";
        return ERR_ARG;
      }
      seen[i] = 1;
    }
    init_special_ = fs;
  }
  reset();
  return OK;
}

void Allocator::reset() {
  free_patch_.assign(init_patch_.begin(), init_patch_.end());
  free_special_.assign(init_special_.begin(), init_special_.end());
  streams_.assign(cfg_.num_streams, StreamState());
}

int Allocator::append(int s, FrameSlots* out, std::string* why) {
  StreamState& st = streams_[s];
  const int64_t pg = cfg_.page_size;
  const int n_s = cfg_.num_special_tokens;
  if (free_patch_.empty() && st.pending.empty()) {
    if (why) *why = "no free patch page (evict, or raise max_patch_pages)";
    return ERR_POOL;
  }
  // special pages this frame opens: one per token landing at slot 0 of a page
  int64_t need = 0;
  for (int j = 0; j < n_s; ++j)
    if ((st.special_tokens + j) % pg == 0) ++need;
  if (need > (int64_t)free_special_.size()) {
    if (why) *why = "special page pool exhausted";
    return ERR_POOL;
  }
  FrameSlots fs;
  // the previous frame is final now: release its held-back window pages
  // (after the checks above, so that an error leaves the state unchanged;
  // the checks count them as free)
  for (int32_t p : st.pending) free_patch_.push_back(p);
  st.pending.clear();
  fs.patch_page = free_patch_.front();
  free_patch_.pop_front();
  st.last_is_live = (int32_t)st.scale_pages.size() >= cfg_.scale_frames;
  if (!st.last_is_live)
    st.scale_pages.push_back(fs.patch_page);
  else
    st.live_pages.push_back(fs.patch_page);
  st.can_rollback = true;
  if (n_s > 0) {
    fs.sp_slot0 = (int32_t)(st.special_tokens % pg);
    if (fs.sp_slot0 != 0) fs.sp_pages[fs.n_sp_pages++] = st.special_pages.back();
    for (int j = 0; j < n_s; ++j) {
      if (st.special_tokens % pg == 0) {
        st.special_pages.push_back(free_special_.front());
        free_special_.pop_front();
        fs.sp_pages[fs.n_sp_pages++] = st.special_pages.back();
      }
      st.special_tokens += 1;
    }
  }
  st.frame_count += 1;
  if (out) *out = fs;
  return OK;
}

int Allocator::evict(int s) {
  StreamState& st = streams_[s];
  int n = 0;
  while ((int32_t)st.live_pages.size() > cfg_.sliding_window) {
    if (defer_)
      st.pending.push_back(st.live_pages.front());
    else
      free_patch_.push_back(st.live_pages.front());
    st.live_pages.pop_front();
    ++n;
  }
  return n;
}

int Allocator::rollback(int s, std::string* why) {
  StreamState& st = streams_[s];
  if (!defer_) {
    if (why) *why = "rollback needs deferred eviction (KVC_OPT_DEFER_EVICTION)";
    return ERR_STATE;
  }
  if (!st.can_rollback || st.frame_count == 0) {
    if (why) *why = "no frame to undo (only the most recent frame, once)";
    return ERR_STATE;
  }
  const int64_t pg = cfg_.page_size;
  const int n_s = cfg_.num_special_tokens;
  // special pages this frame opened, newest first back to the front of the list
  const int64_t before = st.special_tokens - n_s;
  int opened = 0;
  for (int j = 0; j < n_s; ++j)
    if ((before + j) % pg == 0) ++opened;
  for (int i = 0; i < opened; ++i) {
    free_special_.push_front(st.special_pages.back());
    st.special_pages.pop_back();
  }
  st.special_tokens = before;
  if (st.last_is_live) {
    free_patch_.push_front(st.live_pages.back());
    st.live_pages.pop_back();
  } else {
    free_patch_.push_front(st.scale_pages.back());
    st.scale_pages.pop_back();
  }
  while (!st.pending.empty() && (int32_t)st.live_pages.size() < cfg_.sliding_window) {
    st.live_pages.push_front(st.pending.back());
    st.pending.pop_back();
  }
  st.frame_count -= 1;
  st.can_rollback = false;
  return OK;
}

int32_t Allocator::last_page_len(int s) const {
  const StreamState& st = streams_[s];
  if (!st.special_pages.empty())
    return (int32_t)(st.special_tokens - (int64_t)cfg_.page_size * ((int64_t)st.special_pages.size() - 1));
  return cfg_.patch_tokens();
}

// Upper bound of the work units over all planned streams: each stream sees at
// most scale + window patch pages; the special pages are shared out.
static size_t max_units(const Config& c) {
  const size_t upp = (size_t)ceil_div(std::max(1, c.patch_tokens()), KVC_KV_TILE);
  const size_t ups = (size_t)ceil_div(c.page_size, KVC_KV_TILE);
  return (size_t)c.num_streams * (c.scale_frames + c.sliding_window) * upp + (size_t)c.max_special_pages * ups +
         (size_t)c.num_streams;
}

size_t plan_image_ints(const Config& c) {
  // fused plans: at most two more units per own frame and one per stream
  // (the cuts at the special row offset and at each frame's specials), and
  // one pool row per input row
  const size_t own = (size_t)c.num_streams * c.max_frames_per_step;
  return KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * c.num_streams + (size_t)c.max_num_pages() + 4 +
         (size_t)KVC_UNIT_INTS * (max_units(c) + 2 * own + c.num_streams) + 4 +
         (size_t)KVC_MERGE_INTS * KVC_NUM_XCD * c.tiles_capacity() * c.num_heads + 4 + own * c.tokens_per_frame;
}

uint32_t input_row_slot(const Config& c, const FrameSlots& fs, int32_t t) {
  const int32_t off = c.special_row_offset, ns = c.num_special_tokens;
  if (t >= off && t < off + ns) {
    const int32_t pos = fs.sp_slot0 + (t - off);
    const int32_t idx = pos / c.page_size;
    return (uint32_t)fs.sp_pages[idx] * 2u * (uint32_t)c.page_size + (uint32_t)(pos - idx * c.page_size);
  }
  return (uint32_t)fs.patch_page * 2u * (uint32_t)c.page_size + (uint32_t)(t < off ? t : t - ns);
}

namespace {

struct Unit {
  uint32_t slot;   // pool row of the unit's first K row
  int32_t valid;   // rows
  int32_t src;     // fused plans: 1 + the input row of its first row (rows consecutive), 0: pool only
};

// Work units of one stream: 64-slot chunks of each visible page's valid
// slots, in table order.  With `own` (fused plans: the pool row -> input
// row map of the step's own frames, over the pages they touch) a chunk is
// further cut into runs of rows that are either all older (src 0) or all
// own with consecutive input rows.
void stream_units(const Config& c, const int32_t* idx, int32_t n_pages, int32_t n_patch, int32_t last_len,
                  const std::vector<std::pair<int32_t, std::vector<int32_t>>>* own, std::vector<Unit>* out) {
  const int32_t P = c.patch_tokens();
  out->clear();
  for (int32_t pi = 0; pi < n_pages; ++pi) {
    const int32_t len = pi == n_pages - 1 ? last_len : (pi < n_patch ? P : c.page_size);
    const uint32_t base = (uint32_t)idx[pi] * 2u * (uint32_t)c.page_size;
    const std::vector<int32_t>* rows = nullptr;
    if (own)
      for (const auto& pr : *own)
        if (pr.first == idx[pi]) rows = &pr.second;
    for (int32_t a = 0; a < len; a += KVC_KV_TILE) {
      const int32_t b = std::min<int32_t>(len, a + KVC_KV_TILE);
      if (!rows) {
        out->push_back({base + (uint32_t)a, b - a, 0});
        continue;
      }
      int32_t s0 = a;
      while (s0 < b) {
        const int32_t r0 = (*rows)[s0];
        int32_t s1 = s0 + 1;
        while (s1 < b && (r0 < 0 ? (*rows)[s1] < 0 : (*rows)[s1] == r0 + (s1 - s0))) ++s1;
        out->push_back({base + (uint32_t)s0, s1 - s0, r0 < 0 ? 0 : r0 + 1});
        s0 = s1;
      }
    }
  }
}

}  // namespace

void build_plan(const Allocator& a, const std::vector<int32_t>& streams, const std::vector<int32_t>& frames,
                const std::vector<const FrameSlots*>& fslots, const PlanPolicy& pol, HostPlan* out) {
  const Config& c = a.config();
  HostPlan& p = *out;
  const int n = (int)streams.size();
  p.planned = streams;
  p.kv_indptr.assign(1, 0);
  p.kv_indices.clear();
  p.last_page_len.clear();
  p.n_patch_pages.clear();
  p.qo_indptr.assign(1, 0);
  p.n_split.clear();

  const int32_t P = c.patch_tokens();
  std::vector<int64_t> kv_len(n);
  for (int i = 0; i < n; ++i) {
    const StreamState& st = a.stream(streams[i]);
    // [p2] "How LingBot-Map Uses FlashInfer KV Cache for Streaming 3D
    // Reconstruction" §Page Table Planning and Reuse: scale -> window -> specials
    p.kv_indices.insert(p.kv_indices.end(), st.scale_pages.begin(), st.scale_pages.end());
    p.kv_indices.insert(p.kv_indices.end(), st.live_pages.begin(), st.live_pages.end());
    p.kv_indices.insert(p.kv_indices.end(), st.special_pages.begin(), st.special_pages.end());
    p.kv_indptr.push_back((int32_t)p.kv_indices.size());
    const int32_t n_patch = (int32_t)(st.scale_pages.size() + st.live_pages.size());
    p.n_patch_pages.push_back(n_patch);
    p.last_page_len.push_back(a.last_page_len(streams[i]));
    p.qo_indptr.push_back(p.qo_indptr.back() + frames[i] * c.tokens_per_frame);
    kv_len[i] = (int64_t)n_patch * P + st.special_tokens;
  }

  // Work decomposition: each work item is (stream, head, KV split, query
  // group), one work-group.  Every work-group costs about the same per 64-slot
  // unit, its busiest wave's share, so a launch takes as long as its longest
  // split (in units times that per-unit cost) times the number of rounds in
  // which the work-groups run.  The target work-group count is what the
  // device holds at once (one round); the split counts start from each
  // stream's share of it, in proportion to queries x visible tokens, rounded
  // down; then the stream whose splits take longest gains a split while that
  // shortens them and the whole launch still fits in one round.
  double total_work = 0;
  for (int i = 0; i < n; ++i) total_work += (double)frames[i] * (double)kv_len[i];
  // (the float32 kernel runs without splits)
  const int32_t max_splits = c.fp32() ? 1 : std::max(1, std::min<int32_t>(pol.max_splits, KVC_MAX_SPLITS));
  const int32_t upp = (int32_t)ceil_div(std::max(1, P), KVC_KV_TILE);
  const int32_t ups = (int32_t)ceil_div(c.page_size, KVC_KV_TILE);
  // the streams' unit lists (fused plans: cut at the own frames' row runs)
  p.fused = pol.fused;
  std::vector<std::vector<Unit>> ulist(n);
  std::vector<int64_t> units(n), cap(n);
  for (int i = 0; i < n; ++i) {
    std::vector<std::pair<int32_t, std::vector<int32_t>>> own;
    if (p.fused) {
      // input row of every pool slot the step's own frames write, per page
      for (int32_t f = 0; f < frames[i]; ++f)
        for (int32_t t = 0; t < c.tokens_per_frame; ++t) {
          const uint32_t slot = input_row_slot(c, fslots[i][f], t);
          const int32_t page = (int32_t)(slot / (2u * (uint32_t)c.page_size));
          const int32_t j = (int32_t)(slot - (uint32_t)page * 2u * (uint32_t)c.page_size);
          auto it = std::find_if(own.begin(), own.end(), [&](const auto& pr) { return pr.first == page; });
          if (it == own.end()) {
            own.emplace_back(page, std::vector<int32_t>(c.page_size, -1));
            it = own.end() - 1;
          }
          it->second[j] = f * c.tokens_per_frame + t;
        }
    }
    stream_units(c, &p.kv_indices[p.kv_indptr[i]], p.kv_indptr[i + 1] - p.kv_indptr[i], p.n_patch_pages[i],
                 p.last_page_len[i], p.fused ? &own : nullptr, &ulist[i]);
    units[i] = (int64_t)ulist[i].size();
    cap[i] = std::min<int64_t>(max_splits, units[i]);
  }
  // The 32x32 kernel stages a split's unit entries in LDS: at most
  // KVC_MAX_SPLIT_STAGES units per split.
  std::vector<int64_t> min_split32(n, 1), cap32 = cap;
  if (c.tiles32())
    for (int i = 0; i < n; ++i) {
      min_split32[i] = ceil_div(units[i], KVC_MAX_SPLIT_STAGES);
      cap32[i] = std::max(cap[i], min_split32[i]);
    }
  // A query grouping: per stream, its groups, (32x32 kernel) full 32-row
  // tiles and tail, and the per-unit cost of its busiest wave in 16x64
  // tile-steps.
  struct Grouping {
    std::vector<int64_t> n_group, n_t32, tail;
    std::vector<double> per_unit;
    bool variant = false;
    bool k32 = false;   // the 32x32 kernel
  };
  auto grouping = [&](bool variant, bool k32) {
    Grouping g;
    g.variant = variant;
    g.k32 = k32;
    g.n_group.resize(n);
    g.n_t32.assign(n, 0);
    g.tail.assign(n, 0);
    g.per_unit.resize(n);
    for (int i = 0; i < n; ++i) {
      const int64_t n_q = (int64_t)frames[i] * c.tokens_per_frame;
      if (c.fp32()) {
        // float32 kernel: one work-group wave per 16-row query tile
        g.n_group[i] = ceil_div(n_q, KVC_F32_ROWS);
        g.per_unit[i] = 1.0;
      } else if (k32) {
        // variant: rows past the last full 32-row tile, if at most 16, form a
        // tail that the four waves share (a quarter of its slots each)
        const int64_t rem = n_q % KVC_Q_TILE32;
        const bool tail = variant && rem >= 1 && rem <= KVC_TAIL_ROWS;
        const int64_t nt = tail ? n_q / KVC_Q_TILE32 : ceil_div(n_q, KVC_Q_TILE32);
        g.n_group[i] = std::max<int64_t>(1, ceil_div(nt, KVC_GROUP_TILES32));
        g.n_t32[i] = nt;
        g.tail[i] = tail ? 1 : 0;
        // wave w owns tile w of its group and waves w and w + 4 share a SIMD:
        // 2 tile-steps each, plus a quarter tile-step of the tail in every
        // group of a tail launch
        const int64_t kmax = ceil_div(nt, g.n_group[i]);
        g.per_unit[i] = (kmax > 0 ? 2.0 : 0.0) + (kmax > KVC_TAIL_WAVES ? 2.0 : 0.0) + (variant ? 0.25 : 0.0);
      } else {
        // 16x16 kernel: groups of 8 tiles of 16 rows, or 9 with the ninth
        // shared by the four waves (a quarter tile-step each per stage)
        const int64_t nqt = ceil_div(n_q, KVC_Q_TILE);
        g.n_group[i] = ceil_div(nqt, kvc_group_tiles(variant ? 1 : 0));
        g.per_unit[i] = variant ? 2.25 : 2.0;
      }
    }
    return g;
  };
  struct Choice {
    Grouping g;
    std::vector<int64_t> nsplit;
    double cost;
    double length;         // per-unit cost times units of the longest split
    int64_t items_total;   // work-groups of the launch
  };
  // target: the work-groups the device holds at once for the kernel
  auto choose = [&](const Grouping& g, int64_t target) {
    Choice ch;
    ch.g = g;
    ch.nsplit.resize(n);
    std::vector<int64_t> items(n);
    int64_t items_total = 0;
    const std::vector<int64_t>& min_split = g.k32 ? min_split32 : std::vector<int64_t>(n, 1);
    const std::vector<int64_t>& capk = g.k32 ? cap32 : cap;
    for (int i = 0; i < n; ++i) {
      items[i] = (int64_t)c.num_heads * g.n_group[i];
      const double want = total_work > 0 ? (double)target * (double)frames[i] * (double)kv_len[i] /
                                               total_work / (double)items[i]
                                         : 1.0;
      ch.nsplit[i] = std::max<int64_t>(min_split[i], std::min<int64_t>((int64_t)std::floor(want), capk[i]));
      items_total += items[i] * ch.nsplit[i];
    }
    auto length = [&](int i, int64_t ns) { return (double)ceil_div(units[i], ns) * g.per_unit[i]; };
    // The launch lasts as long as the longest split: only that stream's
    // splits are worth adding, and once it cannot gain one (at its cap, over
    // the target, or no shorter for it), no other split would shorten the
    // launch.
    auto longest = [&]() {
      int best = 0;
      for (int i = 1; i < n; ++i)
        if (length(i, ch.nsplit[i]) > length(best, ch.nsplit[best])) best = i;
      return best;
    };
    for (;;) {
      const int b = longest();
      if (ch.nsplit[b] >= capk[b] || items_total + items[b] > target ||
          ceil_div(units[b], ch.nsplit[b] + 1) >= ceil_div(units[b], ch.nsplit[b]))
        break;
      ++ch.nsplit[b];
      items_total += items[b];
    }
    const int64_t rounds = std::max<int64_t>(1, ceil_div(items_total, std::max<int64_t>(1, target)));
    const int b = longest();
    ch.length = length(b, ch.nsplit[b]);
    ch.items_total = items_total;
    ch.cost = ch.length * (double)rounds;
    return ch;
  };
  // Take the grouping variant (a shared tail / a shared ninth tile) when it
  // gives the shorter launch.  At head_dim 64 the 16x16 kernel (up to two
  // work-groups of four waves per CU) competes with the 32x32 one (one of
  // eight, two waves per SIMD).  Its cost is per SIMD too: its per-wave cost
  // times the work-groups that the busiest CU runs (the two resident ones
  // share its SIMDs).  It wins where the 32x32 kernel's groups of 8 tiles of
  // 32 rows spill past one round of work-groups while its own groups of 128
  // rows spread more evenly, as for a multi-frame step over many heads.
  // Only its plain grouping is offered (its shared-tile form does not fit
  // the registers at head_dim 64).
  constexpr double KVC_TILES16_COST = 1.0;   // relative cost of its tile-step
  const int32_t tgt = std::max(1, pol.target_workgroups);
  const bool k32 = c.tiles32();
  Choice ch = choose(grouping(true, k32), tgt);
  p.shared_tile = !c.fp32();
  {
    Choice cand = choose(grouping(false, k32), tgt);
    if (cand.cost < ch.cost) {
      ch = std::move(cand);
      p.shared_tile = false;
    }
  }
  p.tiles16 = false;
  if (k32 && c.head_dim == 64 && pol.query_tile != 32) {
    Choice cand = choose(grouping(false, false), 2 * (int64_t)tgt);
    cand.cost = cand.length * (double)ceil_div(cand.items_total, (int64_t)tgt) * KVC_TILES16_COST;
    if (pol.query_tile == 16 || cand.cost < ch.cost) {
      ch = std::move(cand);
      p.shared_tile = false;
      p.tiles16 = true;
    }
  }
  const std::vector<int64_t>& nsplit = ch.nsplit;

  p.image.assign(KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * n + p.kv_indices.size(), 0);
  int32_t item = 0, tiles = 0;
  p.any_split = false;
  for (int i = 0; i < n; ++i) {
    const int32_t n_q = frames[i] * c.tokens_per_frame;
    const int32_t n_group = (int32_t)ch.g.n_group[i];
    const int64_t ns = nsplit[i];
    p.n_split.push_back((int32_t)ns);
    if (ns > 1) p.any_split = true;

    kvc_dev_stream rec;
    std::memset(&rec, 0, sizeof(rec));
    rec.q_row0 = p.qo_indptr[i];
    rec.n_q = n_q;
    rec.page0 = p.kv_indptr[i];
    rec.n_patch = p.n_patch_pages[i];
    rec.n_pages = p.kv_indptr[i + 1] - p.kv_indptr[i];
    rec.last_len = p.last_page_len[i];
    rec.kv_len = (int32_t)kv_len[i];
    rec.unit0 = 0;   // set below, once the page tables are in place
    rec.n_units = (int32_t)units[i];
    rec.upp = upp;
    rec.ups = ups;
    rec.n_split = (int32_t)ns;
    rec.n_group = n_group;
    rec.q_tile0 = tiles;
    rec.n_t32 = (int32_t)ch.g.n_t32[i];
    rec.tail = (int32_t)ch.g.tail[i];
    tiles += (int32_t)ceil_div(n_q, KVC_Q_TILE32);
    rec.item0 = item;
    rec.n_items = c.num_heads * (int32_t)ns * n_group;
    item += rec.n_items;
    std::memcpy(&p.image[KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * i], &rec, sizeof(rec));
  }
  p.num_items = item;
  p.num_rows = p.qo_indptr.back();
  p.num_tiles = tiles;
  p.image[KVC_HDR_NUM_STREAMS] = n;
  p.image[KVC_HDR_NUM_ITEMS] = item;
  p.image[KVC_HDR_NUM_ROWS] = p.num_rows;
  p.image[KVC_HDR_ANY_SPLIT] = p.any_split ? 1 : 0;
  p.image[KVC_HDR_NUM_TILES] = p.num_tiles;
  p.image[KVC_HDR_SHARED_TILE] = (p.shared_tile ? 1 : 0) | (p.tiles16 ? KVC_VARIANT_TILES16 : 0);
  std::copy(p.kv_indices.begin(), p.kv_indices.end(),
            p.image.begin() + KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * n);

  // Unit tables: the 64-slot chunks of each visible page's valid slots, in
  // table order.  Patch pages hold P valid slots, special pages page_size,
  // the last page last_page_len ([p1] "How FlashInfer KV Cache Attention
  // Accelerates Streaming 3D Reconstruction Over SDPA" §Efficient Attention
  // Masking and Padding: lengths, not masks, delimit the valid tokens).  An
  // entry holds the slot index of the unit's first K row in the block's pool
  // [pages][2][page_size] (below 2^32: validate keeps pages * page_size below
  // 2^31), its valid rows and, in fused plans, 1 + its first input row.
  size_t at = (p.image.size() + 3) & ~(size_t)3;
  for (int i = 0; i < n; ++i) {
    kvc_dev_stream* rec = reinterpret_cast<kvc_dev_stream*>(&p.image[KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * i]);
    kvc_dev_stream r;
    std::memcpy(&r, rec, sizeof(r));
    r.unit0 = (int32_t)at;
    std::memcpy(rec, &r, sizeof(r));
    p.image.resize(at + (size_t)KVC_UNIT_INTS * r.n_units, 0);
    for (int32_t u = 0; u < r.n_units; ++u) {
      const Unit& un = ulist[i][u];
      int32_t* e = &p.image[at + (size_t)KVC_UNIT_INTS * u];
      e[0] = (int32_t)un.slot;
      e[1] = un.valid;
      e[2] = un.src;
      e[3] = 0;
    }
    at += (size_t)KVC_UNIT_INTS * r.n_units;
  }

  // Merge order: the attention work-group of item i runs on XCD
  // i / items_per_xcd (the kernel gives each XCD a contiguous item range), so
  // the split partials of a (tile, head) sit in that XCD's L2.  Each pair of
  // a 32-row tile and a head is merged on the XCD that ran its middle split.
  // An entry carries what the merge needs of its tile (split count and output
  // rows), so that the merge reads one entry before its partials.
  std::vector<std::vector<std::array<int32_t, KVC_MERGE_INTS>>> bucket(KVC_NUM_XCD);
  const int32_t ipx = (p.num_items + KVC_NUM_XCD - 1) / KVC_NUM_XCD;
  for (int i = 0; i < n; ++i) {
    const int32_t n_q = p.qo_indptr[i + 1] - p.qo_indptr[i];
    const int32_t ntile = (int32_t)ceil_div(n_q, KVC_Q_TILE32);
    kvc_dev_stream r;
    std::memcpy(&r, &p.image[KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * i], sizeof(r));
    if (r.n_split <= 1) continue;
    for (int32_t t = 0; t < ntile; ++t) {
      // the query group holding (the first rows of) tile t
      int32_t grp = 0;
      if (k32 && !p.tiles16) {
        if (t >= r.n_t32)
          grp = r.n_group - 1;   // the tail
        else
          while ((grp + 1) * r.n_t32 / r.n_group <= t) ++grp;
      } else {
        const int32_t nqt = (int32_t)ceil_div(n_q, KVC_Q_TILE);
        while ((grp + 1) * nqt / r.n_group <= 2 * t) ++grp;
      }
      for (int32_t h = 0; h < c.num_heads; ++h) {
        const int32_t it = r.item0 + (h * r.n_split + r.n_split / 2) * r.n_group + grp;
        bucket[std::min(it / std::max(1, ipx), KVC_NUM_XCD - 1)].push_back(
            {(r.q_tile0 + t) * c.num_heads + h, r.n_split, p.qo_indptr[i] + KVC_Q_TILE32 * t,
             std::min<int32_t>(KVC_Q_TILE32, n_q - KVC_Q_TILE32 * t)});
      }
    }
  }
  size_t slots = 0;
  for (const auto& b : bucket) slots = std::max(slots, b.size());
  at = (p.image.size() + 3) & ~(size_t)3;
  p.merge_table = (int32_t)at;
  p.merge_slots = (int32_t)slots;
  p.image[KVC_HDR_MERGE_TABLE] = p.merge_table;
  p.image[KVC_HDR_MERGE_SLOTS] = p.merge_slots;
  p.image.resize(at + (size_t)KVC_MERGE_INTS * KVC_NUM_XCD * slots, 0);
  for (int x = 0; x < KVC_NUM_XCD; ++x)
    for (size_t k = 0; k < slots; ++k) {
      int32_t* e = &p.image[at + (size_t)KVC_MERGE_INTS * (x * slots + k)];
      if (k < bucket[x].size())
        std::copy(bucket[x][k].begin(), bucket[x][k].end(), e);
      else
        e[0] = -1;
    }

  // Fused plans: the pool row of each input row (rows in query order: the
  // streams' own frames concatenated), for the copy into the pool.
  p.copy_table = 0;
  if (p.fused) {
    at = (p.image.size() + 3) & ~(size_t)3;
    p.copy_table = (int32_t)at;
    p.image.resize(at + (size_t)p.num_rows, 0);
    for (int i = 0; i < n; ++i)
      for (int32_t f = 0; f < frames[i]; ++f)
        for (int32_t t = 0; t < c.tokens_per_frame; ++t)
          p.image[at + (size_t)p.qo_indptr[i] + (size_t)f * c.tokens_per_frame + t] =
              (int32_t)input_row_slot(c, fslots[i][f], t);
  }
}

}  // namespace kvc
