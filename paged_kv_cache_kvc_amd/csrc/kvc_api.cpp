// C-ABI of the two-stream paged KV cache (declared in include/kvc.h).
//
// Owns host metadata only: the page allocator, the per-step state machine and
// the plan.  Every device buffer (pools, workspace) and the pinned staging
// belong to the caller; the library never allocates device memory.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvc.h"
#include "kvc_host.hpp"
#include "kvc_kernels.h"

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

kvc::Config to_cfg(const kvc_config& c) {
  kvc::Config k;
  k.num_blocks = c.num_blocks;
  k.num_heads = c.num_heads;
  k.head_dim = c.head_dim;
  k.tokens_per_frame = c.tokens_per_frame;
  k.num_special_tokens = c.num_special_tokens;
  k.special_row_offset = c.special_row_offset;
  k.page_size = c.page_size;
  k.scale_frames = c.scale_frames;
  k.sliding_window = c.sliding_window;
  k.num_streams = c.num_streams;
  k.max_patch_pages = c.max_patch_pages;
  k.max_special_pages = c.max_special_pages;
  k.max_frames_per_step = c.max_frames_per_step;
  k.dtype = c.dtype;
  return k;
}

// Workspace layout: [plan 0][plan 1][partial lse][partial o][rotated q],
// 256-byte aligned.
struct Layout {
  size_t plan_bytes, plan0, plan1, lse, part_o, q_rot, total;
};

Layout layout_of(const kvc::Config& c) {
  Layout l;
  l.plan_bytes = align_up(kvc::plan_image_ints(c) * sizeof(int32_t), 256);
  l.plan0 = 0;
  l.plan1 = l.plan_bytes;
  l.lse = 2 * l.plan_bytes;
  // partial outputs are stored per query tile of KVC_Q_TILE32 rows
  const size_t rows = (size_t)c.tiles_capacity() * KVC_Q_TILE32;
  l.part_o = l.lse + align_up((size_t)KVC_MAX_SPLITS * rows * c.num_heads * sizeof(float), 256);
  l.q_rot = l.part_o + align_up((size_t)KVC_MAX_SPLITS * rows * c.num_heads * c.head_dim * sizeof(uint16_t), 256);
  // the step's query rows after the rotary embedding of kvc_run_rope
  l.total = l.q_rot + align_up(rows * c.num_heads * c.head_dim * (size_t)c.elem_bytes(), 256);
  return l;
}

struct EventPair {
  hipEvent_t start, stop;
};

}  // namespace

struct kvc_ctx {
  kvc::Config cfg;
  bool metadata_only = false;
  kvc::Allocator alloc;
  std::vector<void*> pools;
  char* workspace = nullptr;
  char* staging = nullptr;
  Layout lay;

  // per-step state
  bool planned = false;
  bool have_plan = false;
  bool plan_stale = false;            // a rollback happened after this step's plan
  std::vector<uint8_t> advanced;      // [stream]: appended block 0 this step
  std::vector<uint8_t> block_done;    // [stream * num_blocks + block]
  std::vector<int32_t> nframes;       // [stream]: frames appended this step
  std::vector<kvc::FrameSlots> slots; // [stream * max_frames_per_step + f]: this step's frame slots
  kvc::HostPlan plan;
  int plan_buf = 0;
  hipEvent_t staging_done[2] = {nullptr, nullptr};
  bool staging_recorded[2] = {false, false};

  kvc::PlanPolicy policy;
  int cu_count = 256;

  bool profile = false;
  std::vector<EventPair> pending[KVC_NUM_KERNELS];
  std::vector<hipEvent_t> spare;
  double prof_ms[KVC_NUM_KERNELS] = {};
  int64_t prof_n[KVC_NUM_KERNELS] = {};

  std::string err;
};

static kvc_status fail(kvc_ctx* c, kvc_status code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

static kvc_status hip_fail(kvc_ctx* c, int e, const char* what) {
  return fail(c, KVC_ERR_HIP, std::string(what) + ": " + hipGetErrorString((hipError_t)e));
}

static hipEvent_t take_event(kvc_ctx* c) {
  if (!c->spare.empty()) {
    hipEvent_t e = c->spare.back();
    c->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records an event pair around `launch` when profiling is on.
template <class F>
static int timed(kvc_ctx* c, int kernel, void* stream, F launch) {
  if (!c->profile) return launch();
  EventPair ev{take_event(c), take_event(c)};
  if (!ev.start || !ev.stop) return (int)hipErrorOutOfMemory;
  (void)hipEventRecord(ev.start, (hipStream_t)stream);
  const int rc = launch();
  (void)hipEventRecord(ev.stop, (hipStream_t)stream);
  c->pending[kernel].push_back(ev);
  return rc;
}

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_ARG: return "invalid argument";
    case KVC_ERR_STATE: return "call out of order";
    case KVC_ERR_POOL_EXHAUSTED: return "page pool exhausted";
    case KVC_ERR_CAPACITY: return "capacity too small";
    case KVC_ERR_HIP: return "HIP runtime error";
    case KVC_ERR_UNSUPPORTED: return "unsupported shape";
    case KVC_ERR_HOST_ALLOC: return "host memory allocation failed";
    default: return "unknown status";
  }
}

size_t kvc_pool_bytes(const kvc_config* cfg) {
  if (!cfg) return 0;
  const kvc::Config c = to_cfg(*cfg);
  if (kvc::validate(c, nullptr) != kvc::OK) return 0;
  return (size_t)c.max_num_pages() * 2 * c.page_size * c.num_heads * c.head_dim * c.elem_bytes();
}

size_t kvc_workspace_bytes(const kvc_config* cfg) {
  if (!cfg) return 0;
  const kvc::Config c = to_cfg(*cfg);
  if (kvc::validate(c, nullptr) != kvc::OK) return 0;
  return layout_of(c).total;
}

size_t kvc_staging_bytes(const kvc_config* cfg) {
  if (!cfg) return 0;
  const kvc::Config c = to_cfg(*cfg);
  if (kvc::validate(c, nullptr) != kvc::OK) return 0;
  return 2 * layout_of(c).plan_bytes;
}

// Attention work-groups the device holds at once: one per CU (the 32x32
// kernel of head_dim 32 and 64 holds a 128 KiB LDS ring and two waves per
// SIMD; the 16x16 kernel of head_dim 128 one work-group's registers).
static int32_t resident_workgroups(const kvc::Config& c, int cu_count) {
  (void)c;
  return cu_count;
}

static kvc_status create_common_impl(const kvc_config* cfg, const int32_t* fpo, const int32_t* fso, kvc_ctx** out,
                                     kvc_ctx** made);

// Host allocations (page lists, plan vectors) can throw std::bad_alloc; no
// exception may cross the C ABI, so the entry points that allocate turn it
// into KVC_ERR_HOST_ALLOC.
static kvc_status create_common(const kvc_config* cfg, const int32_t* fpo, const int32_t* fso, kvc_ctx** out,
                                kvc_ctx** made) {
  try {
    return create_common_impl(cfg, fpo, fso, out, made);
  } catch (const std::bad_alloc&) {
    return KVC_ERR_HOST_ALLOC;
  }
}

static kvc_status create_common_impl(const kvc_config* cfg, const int32_t* fpo, const int32_t* fso, kvc_ctx** out,
                                     kvc_ctx** made) {
  if (!cfg || !out) return KVC_ERR_ARG;
  *out = nullptr;
  kvc::Config c = to_cfg(*cfg);
  std::string why;
  const int v = kvc::validate(c, &why);
  if (v != kvc::OK) return (kvc_status)v;
  kvc_ctx* x = new (std::nothrow) kvc_ctx();
  if (!x) return KVC_ERR_HOST_ALLOC;
  try {
    x->cfg = c;
    std::vector<int32_t> fp, fs;
    if (fpo) fp.assign(fpo, fpo + c.max_patch_pages);
    if (fso) fs.assign(fso, fso + c.max_special_pages);
    if (fso && c.max_special_pages == 0) fs.clear();
    const int rc = x->alloc.init(c, fp, fs, &why);
    if (rc != kvc::OK) {
      delete x;
      return (kvc_status)rc;
    }
    x->advanced.assign(c.num_streams, 0);
    x->block_done.assign((size_t)c.num_streams * c.num_blocks, 0);
    x->slots.assign((size_t)c.num_streams * c.max_frames_per_step, kvc::FrameSlots());
    x->nframes.assign(c.num_streams, 0);
    x->lay = layout_of(c);
  } catch (const std::bad_alloc&) {
    delete x;
    return KVC_ERR_HOST_ALLOC;
  }
  *made = x;
  return KVC_OK;
}

kvc_status kvc_create_metadata_only(const kvc_config* cfg, const int32_t* fpo, const int32_t* fso, kvc_ctx** out) {
  kvc_ctx* x = nullptr;
  const kvc_status rc = create_common(cfg, fpo, fso, out, &x);
  if (rc != KVC_OK) return rc;
  x->metadata_only = true;
  x->policy.target_workgroups = resident_workgroups(x->cfg, x->cu_count);
  *out = x;
  return KVC_OK;
}

kvc_status kvc_create(const kvc_config* cfg, void* const* pools, void* workspace, void* staging,
                      const int32_t* fpo, const int32_t* fso, kvc_ctx** out) {
  if (!pools || !workspace || !staging) return KVC_ERR_ARG;
  if (((uintptr_t)workspace & 255) != 0) return KVC_ERR_ARG;
  kvc_ctx* x = nullptr;
  const kvc_status rc = create_common(cfg, fpo, fso, out, &x);
  if (rc != KVC_OK) return rc;
  const size_t pb = kvc_pool_bytes(cfg);
  for (int b = 0; b < x->cfg.num_blocks; ++b) {
    if (!pools[b] || ((uintptr_t)pools[b] & 15) != 0) {
      delete x;
      return KVC_ERR_ARG;
    }
    x->pools.push_back(pools[b]);
  }
  x->workspace = static_cast<char*>(workspace);
  x->staging = static_cast<char*>(staging);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&x->cu_count, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    delete x;
    return KVC_ERR_HIP;
  }
  x->policy.target_workgroups = resident_workgroups(x->cfg, x->cu_count);
  for (int b = 0; b < x->cfg.num_blocks; ++b) {
    if (hipMemset(x->pools[b], 0, pb) != hipSuccess) {
      delete x;
      return KVC_ERR_HIP;
    }
  }
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&x->staging_done[i], hipEventDisableTiming) != hipSuccess) {
      delete x;
      return KVC_ERR_HIP;
    }
  }
  *out = x;
  return KVC_OK;
}

kvc_status kvc_destroy(kvc_ctx* c) {
  if (!c) return KVC_ERR_ARG;
  if (!c->metadata_only) {
    for (int i = 0; i < 2; ++i)
      if (c->staging_done[i]) {
        (void)hipEventSynchronize(c->staging_done[i]);
        (void)hipEventDestroy(c->staging_done[i]);
      }
    for (int k = 0; k < KVC_NUM_KERNELS; ++k)
      for (auto& e : c->pending[k]) {
        (void)hipEventSynchronize(e.stop);
        (void)hipEventDestroy(e.start);
        (void)hipEventDestroy(e.stop);
      }
    for (auto e : c->spare) (void)hipEventDestroy(e);
  }
  delete c;
  return KVC_OK;
}

kvc_status kvc_reset(kvc_ctx* c) {
  if (!c) return KVC_ERR_ARG;
  c->alloc.reset();
  // every per-step field: the next call must be a block-0 append
  c->planned = false;
  c->have_plan = false;
  c->plan_stale = false;
  std::fill(c->advanced.begin(), c->advanced.end(), 0);
  std::fill(c->block_done.begin(), c->block_done.end(), 0);
  std::fill(c->nframes.begin(), c->nframes.end(), 0);
  std::fill(c->slots.begin(), c->slots.end(), kvc::FrameSlots());
  c->plan = kvc::HostPlan();
  c->err.clear();
  return KVC_OK;
}

static kvc_status append_frames_impl(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                                     int32_t num_frames, const float* rope_cos, const float* rope_sin, bool rope,
                                     kvc_stream_t hs);
static kvc_status launch_appends(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                                 int32_t num_frames, const float* rope_cos, const float* rope_sin, bool rope,
                                 kvc_stream_t hs);

// Some block's append of this step waits for its kvc_run_append.
static bool deferred_pending(const kvc_ctx* c) {
  for (uint8_t d : c->block_done)
    if (d == 2) return true;
  return false;
}

kvc_status kvc_append_frames(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                             int32_t num_frames, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  try {
    return append_frames_impl(c, stream, block, k, v, num_frames, nullptr, nullptr, false, hs);
  } catch (const std::bad_alloc&) {
    return fail(c, KVC_ERR_HOST_ALLOC, "host allocation failed");
  }
}

kvc_status kvc_append_frames_rope(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                                  int32_t num_frames, const float* rope_cos, const float* rope_sin,
                                  kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  try {
    return append_frames_impl(c, stream, block, k, v, num_frames, rope_cos, rope_sin, true, hs);
  } catch (const std::bad_alloc&) {
    return fail(c, KVC_ERR_HOST_ALLOC, "host allocation failed");
  }
}

static bool table_ok(const float* t) { return t && ((uintptr_t)t & 15) == 0; }

static kvc_status append_frames_impl(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                                     int32_t num_frames, const float* rope_cos, const float* rope_sin, bool rope,
                                     kvc_stream_t hs) {
  const kvc::Config& cf = c->cfg;
  if (stream < 0 || stream >= cf.num_streams) return fail(c, KVC_ERR_ARG, "stream out of range");
  if (block < 0 || block >= cf.num_blocks) return fail(c, KVC_ERR_ARG, "block out of range");
  if (num_frames < 1 || num_frames > cf.max_frames_per_step)
    return fail(c, KVC_ERR_ARG, "num_frames must be in [1, max_frames_per_step]");
  // k = v = NULL on a device context: the copy is deferred to this block's
  // kvc_run_append (KVC_OPT_FUSED_APPEND only)
  const bool deferred = !c->metadata_only && !k && !v && !rope;
  if (c->metadata_only) {
    if (k || v || rope_cos || rope_sin)
      return fail(c, KVC_ERR_ARG, "metadata-only context takes k = v = NULL and no rotary tables");
  } else if (deferred) {
    if (!c->policy.fused)
      return fail(c, KVC_ERR_ARG, "k = v = NULL defers the copy, which needs KVC_OPT_FUSED_APPEND");
  } else if (!k || !v || ((uintptr_t)k & 15) || ((uintptr_t)v & 15)) {
    return fail(c, KVC_ERR_ARG, "k and v must be 16-byte aligned device pointers");
  } else if (rope && (!table_ok(rope_cos) || !table_ok(rope_sin))) {
    return fail(c, KVC_ERR_ARG, "rope_cos and rope_sin must be 16-byte aligned device pointers");
  }
  const size_t bd = (size_t)stream * cf.num_blocks + block;
  kvc::FrameSlots* fs = &c->slots[(size_t)stream * cf.max_frames_per_step];
  if (block == 0) {
    // kvc_plan ends a step; the first block-0 append after it starts the next.
    const bool new_step = c->planned;
    if (new_step && deferred_pending(c))
      return fail(c, KVC_ERR_STATE, "a deferred append of the last step was not completed by kvc_run_append");
    if (!new_step && c->advanced[stream])
      return fail(c, KVC_ERR_STATE, "stream already appended block 0 this step (kvc_plan ends a step)");
    std::string why;
    if (num_frames == 1) {
      const int rc = c->alloc.append(stream, &fs[0], &why);
      if (rc != kvc::OK) return fail(c, (kvc_status)rc, why);
    } else {
      // all frames or none
      const kvc::Allocator before = c->alloc;
      for (int32_t f = 0; f < num_frames; ++f) {
        const int rc = c->alloc.append(stream, &fs[f], &why);
        if (rc != kvc::OK) {
          c->alloc = before;
          return fail(c, (kvc_status)rc, why);
        }
      }
    }
    if (new_step) {
      c->planned = false;
      std::fill(c->advanced.begin(), c->advanced.end(), 0);
      std::fill(c->block_done.begin(), c->block_done.end(), 0);
    }
    c->advanced[stream] = 1;
    c->nframes[stream] = num_frames;
  } else {
    if (!c->advanced[stream]) return fail(c, KVC_ERR_STATE, "append of block >= 1 before block 0 in this step");
    if (c->block_done[bd]) return fail(c, KVC_ERR_STATE, "block already appended for this stream in this step");
    if (num_frames != c->nframes[stream])
      return fail(c, KVC_ERR_ARG, "num_frames differs from this step's block-0 append");
  }
  c->block_done[bd] = deferred ? 2 : 1;
  if (c->metadata_only || deferred) return KVC_OK;
  return launch_appends(c, stream, block, k, v, num_frames, rope_cos, rope_sin, rope, hs);
}

// The append kernels of one stream's frames of this step into a block's pool.
static kvc_status launch_appends(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                                 int32_t num_frames, const float* rope_cos, const float* rope_sin, bool rope,
                                 kvc_stream_t hs) {
  const kvc::Config& cf = c->cfg;
  const kvc::FrameSlots* fs = &c->slots[(size_t)stream * cf.max_frames_per_step];
  const size_t frame_bytes = (size_t)cf.tokens_per_frame * cf.num_heads * cf.head_dim * cf.elem_bytes();
  const size_t frame_table = (size_t)cf.tokens_per_frame * (cf.head_dim / 2);
  for (int32_t f = 0; f < num_frames; ++f) {
    kvc::AppendParams p;
    std::memset(&p, 0, sizeof(p));
    p.pool = c->pools[block];
    p.k = static_cast<const char*>(k) + f * frame_bytes;
    p.v = static_cast<const char*>(v) + f * frame_bytes;
    if (rope) {
      p.rope_cos = rope_cos + f * frame_table;
      p.rope_sin = rope_sin + f * frame_table;
    }
    p.head_dim = cf.head_dim;
    p.dtype = cf.dtype;
    p.T = cf.tokens_per_frame;
    p.row_elems = cf.num_heads * cf.head_dim;
    p.elem_bytes = cf.elem_bytes();
    p.special_row_offset = cf.special_row_offset;
    p.n_special = cf.num_special_tokens;
    p.page_size = cf.page_size;
    p.patch_page = fs[f].patch_page;
    p.sp_slot0 = fs[f].sp_slot0;
    p.n_sp_pages = fs[f].n_sp_pages;
    for (int i = 0; i < KVC_MAX_APPEND_SPECIAL_PAGES; ++i) p.sp_pages[i] = fs[f].sp_pages[i];
    const int e = timed(c, KVC_KERNEL_APPEND, hs, [&] { return kvc::launch_append(p, hs); });
    if (e) return hip_fail(c, e, "append launch");
  }
  return KVC_OK;
}

kvc_status kvc_append_frame(kvc_ctx* c, int32_t stream, int32_t block, const void* k, const void* v,
                            kvc_stream_t hs) {
  return kvc_append_frames(c, stream, block, k, v, 1, hs);
}

kvc_status kvc_rollback(kvc_ctx* c, int32_t stream) {
  if (!c) return KVC_ERR_ARG;
  if (stream < 0 || stream >= c->cfg.num_streams) return fail(c, KVC_ERR_ARG, "stream out of range");
  bool mid_step = false;
  for (uint8_t a : c->advanced) mid_step = mid_step || a;
  if (mid_step && !c->planned) return fail(c, KVC_ERR_STATE, "rollback inside a step (call it after kvc_plan)");
  if (deferred_pending(c))
    return fail(c, KVC_ERR_STATE, "rollback with a deferred append pending (complete it with kvc_run_append)");
  std::string why;
  const int rc = c->alloc.rollback(stream, &why);
  if (rc != kvc::OK) return fail(c, (kvc_status)rc, why);
  c->plan_stale = true;
  return KVC_OK;
}

kvc_status kvc_evict(kvc_ctx* c, int32_t stream) {
  if (!c) return KVC_ERR_ARG;
  if (stream < 0 || stream >= c->cfg.num_streams) return fail(c, KVC_ERR_ARG, "stream out of range");
  c->alloc.evict(stream);
  return KVC_OK;
}

static kvc_status plan_impl(kvc_ctx* c, kvc_stream_t hs);

kvc_status kvc_plan(kvc_ctx* c, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  try {
    return plan_impl(c, hs);
  } catch (const std::bad_alloc&) {
    return fail(c, KVC_ERR_HOST_ALLOC, "host allocation failed");
  }
}

static kvc_status plan_impl(kvc_ctx* c, kvc_stream_t hs) {
  if (c->planned) return fail(c, KVC_ERR_STATE, "already planned this step");
  std::vector<int32_t> streams, frames;
  for (int s = 0; s < c->cfg.num_streams; ++s)
    if (c->advanced[s]) {
      streams.push_back(s);
      frames.push_back(c->nframes[s]);
    }
  if (streams.empty()) return fail(c, KVC_ERR_STATE, "no stream appended block 0 this step");
  std::vector<const kvc::FrameSlots*> fslots;
  for (int32_t s : streams) fslots.push_back(&c->slots[(size_t)s * c->cfg.max_frames_per_step]);
  kvc::HostPlan next;
  kvc::build_plan(c->alloc, streams, frames, fslots, c->policy, &next);
  // The device plan buffer (and its staging half) holds plan_image_ints ints,
  // enough while every planned stream sees at most scale_frames +
  // sliding_window patch pages.  A stream whose window was not evicted can
  // exceed it; refuse such a plan rather than overrun the buffers.
  if (next.image.size() > kvc::plan_image_ints(c->cfg))
    return fail(c, KVC_ERR_CAPACITY,
                "plan larger than the plan buffer: a planned stream holds more than scale_frames + "
                "sliding_window patch pages (call kvc_evict before kvc_plan)");
  // The split partial buffers hold KVC_MAX_SPLITS splits; up to head_dim 64
  // a split covers at most KVC_MAX_SPLIT_STAGES units (its LDS entry table).
  for (int32_t ns : next.n_split)
    if (ns > KVC_MAX_SPLITS)
      return fail(c, KVC_ERR_CAPACITY,
                  "a planned stream sees more than " + std::to_string(KVC_MAX_SPLITS * KVC_MAX_SPLIT_STAGES * 64) +
                      " tokens (64 splits of 512 units of 64 slots)");
  c->plan = std::move(next);
  c->planned = true;
  c->plan_stale = false;
  c->have_plan = true;
  if (c->metadata_only) return KVC_OK;

  const int b = c->plan_buf ^ 1;
  if (c->staging_recorded[b]) {
    const hipError_t e = hipEventSynchronize(c->staging_done[b]);
    if (e != hipSuccess) return hip_fail(c, e, "plan staging wait");
  }
  const size_t bytes = c->plan.image.size() * sizeof(int32_t);
  if (bytes > c->lay.plan_bytes) return fail(c, KVC_ERR_CAPACITY, "plan image exceeds the plan buffer");
  char* host = c->staging + b * c->lay.plan_bytes;
  std::memcpy(host, c->plan.image.data(), bytes);
  char* dev = c->workspace + (b ? c->lay.plan1 : c->lay.plan0);
  hipError_t e = hipMemcpyAsync(dev, host, bytes, hipMemcpyHostToDevice, (hipStream_t)hs);
  if (e != hipSuccess) return hip_fail(c, e, "plan upload");
  e = hipEventRecord(c->staging_done[b], (hipStream_t)hs);
  if (e != hipSuccess) return hip_fail(c, e, "plan upload event");
  c->staging_recorded[b] = true;
  c->plan_buf = b;
  return KVC_OK;
}

// Checks and launches of one block's attention (and merge), with the split
// partials at lse / po.  `partials` says where they live, for messages.
static kvc_status check_run(kvc_ctx* c, int32_t block, const void* q, const void* o) {
  if (c->metadata_only) return fail(c, KVC_ERR_STATE, "metadata-only context cannot run");
  const kvc::Config& cf = c->cfg;
  if (block < 0 || block >= cf.num_blocks) return fail(c, KVC_ERR_ARG, "block out of range");
  if (!q || !o || ((uintptr_t)q & 15) || ((uintptr_t)o & 15)) return fail(c, KVC_ERR_ARG, "q and o must be 16-byte aligned");
  if (q == o) return fail(c, KVC_ERR_ARG, "o must not alias q");
  if (!c->planned) return fail(c, KVC_ERR_STATE, "run before plan in this step");
  if (c->plan_stale) return fail(c, KVC_ERR_STATE, "a rollback since the plan: append and plan the next step first");
  for (int32_t s : c->plan.planned) {
    const uint8_t d = c->block_done[(size_t)s * cf.num_blocks + block];
    if (d == 2) return fail(c, KVC_ERR_STATE, "a planned stream deferred this block's append: use kvc_run_append");
    if (d != 1) return fail(c, KVC_ERR_STATE, "a planned stream has not appended this block");
  }
  return KVC_OK;
}

// Inputs of a fused run: per planned stream (plan order) its k and v rows.
struct FusedInputs {
  const void* k[KVC_ARG_STREAMS];
  const void* v[KVC_ARG_STREAMS];
};

static kvc_status launch_run(kvc_ctx* c, int32_t block, const void* q, void* o, kvc_stream_t hs, float* lse,
                             void* po, const FusedInputs* fin = nullptr) {
  const kvc::Config& cf = c->cfg;
  const int32_t* dplan = reinterpret_cast<const int32_t*>(c->workspace + (c->plan_buf ? c->lay.plan1 : c->lay.plan0));

  kvc::AttnParams a;
  std::memset(&a, 0, sizeof(a));
  a.plan = dplan;
  a.pool = c->pools[block];
  a.q = q;
  a.o = o;
  a.part_o = po;
  a.part_lse = lse;
  a.num_heads = cf.num_heads;
  a.head_dim = cf.head_dim;
  a.page_size = cf.page_size;
  a.patch_tokens = cf.patch_tokens();
  a.tiles_cap = cf.tiles_capacity();
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cf.head_dim));
  a.num_items = c->plan.num_items;
  a.dtype = cf.dtype;
  a.items_per_xcd = (c->plan.num_items + 7) / 8;
  a.shared_tile = c->plan.shared_tile ? 1 : 0;
  a.num_streams = (int32_t)c->plan.planned.size();
  if (a.num_streams <= KVC_ARG_STREAMS)
    std::memcpy(a.recs, c->plan.image.data() + KVC_PLAN_HEADER_INTS, (size_t)a.num_streams * sizeof(kvc_dev_stream));
  if (fin) {
    a.fused = 1;
    for (int i = 0; i < a.num_streams; ++i) {
      a.kin[i] = fin->k[i];
      a.vin[i] = fin->v[i];
    }
  }
  const int32_t grid = 8 * a.items_per_xcd;
  int e = timed(c, KVC_KERNEL_ATTENTION, hs, [&] {
    if (cf.fp32()) return kvc::launch_attention_f32(a, hs);
    return cf.tiles32() && !c->plan.tiles16 ? kvc::launch_attention32(a, grid, hs)
                                            : kvc::launch_attention(a, grid, hs);
  });
  if (e) return hip_fail(c, e, "attention launch");
  if (c->plan.any_split) {
    kvc::MergeParams m;
    std::memset(&m, 0, sizeof(m));
    m.plan = dplan;
    m.part_o = po;
    m.part_lse = lse;
    m.o = o;
    m.num_heads = cf.num_heads;
    m.head_dim = cf.head_dim;
    m.tiles_cap = cf.tiles_capacity();
    m.num_tiles = c->plan.num_tiles;
    m.max_split = *std::max_element(c->plan.n_split.begin(), c->plan.n_split.end());
    m.merge_table = c->plan.merge_table;
    m.merge_slots = c->plan.merge_slots;
    m.dtype = cf.dtype;
    if (fin) {
      // the copy of the step's rows into the pool rides on the merge launch
      m.copy_rows = c->plan.num_rows;
      m.row_bytes = cf.num_heads * cf.head_dim * cf.elem_bytes();
      const int64_t copies = (int64_t)m.copy_rows * 2 * (m.row_bytes / 16);
      const int64_t per_wg = (int64_t)KVC_COPY_PER * 64 * (cf.head_dim / 32) * 4;
      m.copy_wgs = (int32_t)((copies + per_wg - 1) / per_wg);
      m.copy_table = c->plan.copy_table;
      m.page_size = cf.page_size;
      m.num_streams = a.num_streams;
      for (int i = 0; i <= a.num_streams; ++i) m.row0[i] = c->plan.qo_indptr[i];
      m.pool = c->pools[block];
      for (int i = 0; i < a.num_streams; ++i) {
        m.kin[i] = fin->k[i];
        m.vin[i] = fin->v[i];
      }
    }
    e = timed(c, KVC_KERNEL_MERGE, hs, [&] { return kvc::launch_merge(m, hs); });
    if (e) return hip_fail(c, e, "merge launch");
  }
  return KVC_OK;
}

kvc_status kvc_run(kvc_ctx* c, int32_t block, const void* q, void* o, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  const kvc_status rc = check_run(c, block, q, o);
  if (rc != KVC_OK) return rc;
  return launch_run(c, block, q, o, hs, reinterpret_cast<float*>(c->workspace + c->lay.lse),
                    c->workspace + c->lay.part_o);
}

kvc_status kvc_run_append(kvc_ctx* c, int32_t block, const void* const* k, const void* const* v, const void* q,
                          void* o, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  const kvc::Config& cf = c->cfg;
  if (c->metadata_only) return fail(c, KVC_ERR_STATE, "metadata-only context cannot run");
  if (block < 0 || block >= cf.num_blocks) return fail(c, KVC_ERR_ARG, "block out of range");
  if (!k || !v) return fail(c, KVC_ERR_ARG, "k and v must be arrays of num_streams device pointers");
  if (!q || !o || ((uintptr_t)q & 15) || ((uintptr_t)o & 15)) return fail(c, KVC_ERR_ARG, "q and o must be 16-byte aligned");
  if (q == o) return fail(c, KVC_ERR_ARG, "o must not alias q");
  if (!c->planned) return fail(c, KVC_ERR_STATE, "run before plan in this step");
  if (c->plan_stale) return fail(c, KVC_ERR_STATE, "a rollback since the plan: append and plan the next step first");
  if (!c->plan.fused) return fail(c, KVC_ERR_STATE, "the plan was built without KVC_OPT_FUSED_APPEND");
  for (int32_t s : c->plan.planned) {
    const uint8_t d = c->block_done[(size_t)s * cf.num_blocks + block];
    if (d == 1) return fail(c, KVC_ERR_STATE, "a planned stream already appended this block (use kvc_run)");
    if (d == 0 && block == 0) return fail(c, KVC_ERR_STATE, "block 0 is appended (or deferred) before the plan");
    if (!k[s] || !v[s] || ((uintptr_t)k[s] & 15) || ((uintptr_t)v[s] & 15))
      return fail(c, KVC_ERR_ARG, "k[s] and v[s] of a planned stream must be 16-byte aligned device pointers");
  }
  for (int32_t s : c->plan.planned) c->block_done[(size_t)s * cf.num_blocks + block] = 1;
  float* lse = reinterpret_cast<float*>(c->workspace + c->lay.lse);
  char* po = c->workspace + c->lay.part_o;
  const int n = (int)c->plan.planned.size();
  // One attention launch reading the own rows from k / v and one merge
  // launch that also copies them into the pool: 32x32 kernel, split plans,
  // at most KVC_ARG_STREAMS streams.  Otherwise the appends, then the run.
  if (!cf.fp32() && cf.tiles32() && !c->plan.tiles16 && c->plan.any_split && n <= KVC_ARG_STREAMS) {
    FusedInputs fin;
    std::memset(&fin, 0, sizeof(fin));
    for (int i = 0; i < n; ++i) {
      fin.k[i] = k[c->plan.planned[i]];
      fin.v[i] = v[c->plan.planned[i]];
    }
    return launch_run(c, block, q, o, hs, lse, po, &fin);
  }
  for (int i = 0; i < n; ++i) {
    const int32_t s = c->plan.planned[i];
    const kvc_status rc = launch_appends(c, s, block, k[s], v[s], c->nframes[s], nullptr, nullptr, false, hs);
    if (rc != KVC_OK) return rc;
  }
  return launch_run(c, block, q, o, hs, lse, po);
}

kvc_status kvc_run_rope(kvc_ctx* c, int32_t block, const void* q, const float* rope_cos, const float* rope_sin,
                        void* o, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  kvc_status rc = check_run(c, block, q, o);
  if (rc != KVC_OK) return rc;
  if (!table_ok(rope_cos) || !table_ok(rope_sin))
    return fail(c, KVC_ERR_ARG, "rope_cos and rope_sin must be 16-byte aligned device pointers");
  const kvc::Config& cf = c->cfg;
  void* qr = c->workspace + c->lay.q_rot;
  kvc::RopeParams r;
  std::memset(&r, 0, sizeof(r));
  r.x = q;
  r.y = qr;
  r.cos = rope_cos;
  r.sin = rope_sin;
  r.row_elems = cf.num_heads * cf.head_dim;
  r.head_dim = cf.head_dim;
  r.dtype = cf.dtype;
  r.chunks = (int64_t)c->plan.qo_indptr.back() * r.row_elems * cf.elem_bytes() / 16;
  if (r.chunks >= ((int64_t)1 << 31)) return fail(c, KVC_ERR_UNSUPPORTED, "more than 2^31 query chunks");
  const int e = timed(c, KVC_KERNEL_ROPE, hs, [&] { return kvc::launch_rope(r, hs); });
  if (e) return hip_fail(c, e, "rope launch");
  return launch_run(c, block, qr, o, hs, reinterpret_cast<float*>(c->workspace + c->lay.lse),
                    c->workspace + c->lay.part_o);
}

// Bytes of split partials one plan writes, laid out as in the workspace
// ([split][head][query tile] lse rows, then the outputs), for the plan's
// largest split count rather than the workspace's maximum.
static void partial_extent(const kvc::Config& cf, int32_t max_split, size_t* lse_bytes, size_t* total) {
  const size_t rows = (size_t)cf.tiles_capacity() * KVC_Q_TILE32;
  *lse_bytes = align_up((size_t)max_split * rows * cf.num_heads * sizeof(float), 256);
  *total = *lse_bytes + (size_t)max_split * rows * cf.num_heads * cf.head_dim * sizeof(uint16_t);
}

kvc_status kvc_run_no_alloc(kvc_ctx* c, int32_t block, const void* q, void* o, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  const kvc_status rc = check_run(c, block, q, o);
  if (rc != KVC_OK) return rc;
  char* base = nullptr;
  size_t cap = 0;
  const int e = kvc::no_alloc_scratch(reinterpret_cast<void**>(&base), &cap);
  if (e) return hip_fail(c, e, "static scratch address");
  const int32_t max_split = *std::max_element(c->plan.n_split.begin(), c->plan.n_split.end());
  size_t lse_bytes = 0, need = 0;
  partial_extent(c->cfg, max_split, &lse_bytes, &need);
  if (need > cap)
    return fail(c, KVC_ERR_CAPACITY,
                "the step's split partials need " + std::to_string(need) + " bytes, above the static scratch's " +
                    std::to_string(cap) + " (fewer splits via KVC_OPT_MAX_SPLITS, or kvc_run)");
  // with max_split splits the partial tiles are indexed exactly as in the
  // workspace layout, only with the plan's split count as the extent
  return launch_run(c, block, q, o, hs, reinterpret_cast<float*>(base), base + lse_bytes);
}

kvc_status kvc_get_plan(const kvc_ctx* c, int32_t* planned, int32_t* kv_indptr, int32_t* kv_indices,
                        int32_t* last_page_len, int32_t* n_patch_pages, int32_t* qo_indptr, int32_t* n_splits,
                        int32_t cap_streams, int32_t cap_indices, int32_t* num_planned, int32_t* num_indices) {
  if (!c) return KVC_ERR_ARG;
  kvc_ctx* m = const_cast<kvc_ctx*>(c);
  if (!c->have_plan) return fail(m, KVC_ERR_STATE, "no plan");
  const kvc::HostPlan& p = c->plan;
  const int32_t n = (int32_t)p.planned.size();
  const int32_t ni = (int32_t)p.kv_indices.size();
  if (num_planned) *num_planned = n;
  if (num_indices) *num_indices = ni;
  if ((planned || kv_indptr || last_page_len || n_patch_pages || qo_indptr || n_splits) && cap_streams < n)
    return fail(m, KVC_ERR_ARG, "capacity_streams too small");
  if (kv_indices && cap_indices < ni) return fail(m, KVC_ERR_ARG, "capacity_indices too small");
  if (planned) std::copy(p.planned.begin(), p.planned.end(), planned);
  if (kv_indptr) std::copy(p.kv_indptr.begin(), p.kv_indptr.end(), kv_indptr);
  if (kv_indices) std::copy(p.kv_indices.begin(), p.kv_indices.end(), kv_indices);
  if (last_page_len) std::copy(p.last_page_len.begin(), p.last_page_len.end(), last_page_len);
  if (n_patch_pages) std::copy(p.n_patch_pages.begin(), p.n_patch_pages.end(), n_patch_pages);
  if (qo_indptr) std::copy(p.qo_indptr.begin(), p.qo_indptr.end(), qo_indptr);
  if (n_splits) std::copy(p.n_split.begin(), p.n_split.end(), n_splits);
  return KVC_OK;
}

kvc_status kvc_get_plan_shape(const kvc_ctx* c, int32_t* work_items, int32_t* group_rows) {
  if (!c) return KVC_ERR_ARG;
  if (!c->have_plan) return fail(const_cast<kvc_ctx*>(c), KVC_ERR_STATE, "no plan");
  if (work_items) *work_items = c->plan.num_items;
  if (group_rows) {
    if (c->cfg.fp32())
      *group_rows = KVC_F32_ROWS;
    else if (c->cfg.tiles32() && !c->plan.tiles16)
      *group_rows = KVC_GROUP_TILES32 * KVC_Q_TILE32 + (c->plan.shared_tile ? KVC_TAIL_ROWS : 0);
    else
      *group_rows = kvc_group_tiles(c->plan.shared_tile ? 1 : 0) * KVC_Q_TILE;
  }
  return KVC_OK;
}

kvc_status kvc_get_plan_image(const kvc_ctx* c, int32_t* buf, int32_t capacity, int32_t* n_ints) {
  if (!c) return KVC_ERR_ARG;
  kvc_ctx* m = const_cast<kvc_ctx*>(c);
  if (!c->have_plan) return fail(m, KVC_ERR_STATE, "no plan");
  const int32_t n = (int32_t)c->plan.image.size();
  if (n_ints) *n_ints = n;
  if (buf) {
    if (capacity < n) return fail(m, KVC_ERR_ARG, "capacity too small");
    std::copy(c->plan.image.begin(), c->plan.image.end(), buf);
  }
  return KVC_OK;
}

kvc_status kvc_get_split_partials(const kvc_ctx* c, float* lse, int64_t cap_lse, uint16_t* o, int64_t cap_o,
                                  int64_t* n_lse, int64_t* n_o, kvc_stream_t hs) {
  if (!c) return KVC_ERR_ARG;
  kvc_ctx* m = const_cast<kvc_ctx*>(c);
  if (!c->have_plan) return fail(m, KVC_ERR_STATE, "no plan");
  const size_t rows = (size_t)c->cfg.tiles_capacity() * KVC_Q_TILE32;
  const int64_t nl = (int64_t)KVC_MAX_SPLITS * (int64_t)rows * c->cfg.num_heads;
  const int64_t no = nl * c->cfg.head_dim;
  if (n_lse) *n_lse = nl;
  if (n_o) *n_o = no;
  if ((lse && cap_lse < nl) || (o && cap_o < no)) return fail(m, KVC_ERR_ARG, "capacity too small");
  if (c->metadata_only) return fail(m, KVC_ERR_STATE, "metadata-only context has no device buffers");
  hipError_t e = hipStreamSynchronize((hipStream_t)hs);
  if (e == hipSuccess && lse)
    e = hipMemcpy(lse, c->workspace + c->lay.lse, (size_t)nl * sizeof(float), hipMemcpyDeviceToHost);
  if (e == hipSuccess && o)
    e = hipMemcpy(o, c->workspace + c->lay.part_o, (size_t)no * sizeof(uint16_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(m, e, "copy of the split partials");
  return KVC_OK;
}

kvc_status kvc_get_stats(const kvc_ctx* c, int32_t stream, kvc_stats* out) {
  if (!c || !out) return KVC_ERR_ARG;
  if (stream < 0 || stream >= c->cfg.num_streams) return KVC_ERR_ARG;
  const kvc::StreamState& st = c->alloc.stream(stream);
  std::memset(out, 0, sizeof(*out));
  out->frame_count = st.frame_count;
  out->special_tokens = st.special_tokens;
  out->scale_pages = (int32_t)st.scale_pages.size();
  out->live_pages = (int32_t)st.live_pages.size();
  out->free_pages = c->alloc.free_patch_count();
  out->special_pages = (int32_t)st.special_pages.size();
  out->free_special_pages = c->alloc.free_special_count();
  return KVC_OK;
}

kvc_status kvc_set_option(kvc_ctx* c, int32_t option, int64_t value) {
  if (!c) return KVC_ERR_ARG;
  switch (option) {
    case KVC_OPT_TARGET_WORKGROUPS:
      if (value < 1 || value > (1 << 20)) return fail(c, KVC_ERR_ARG, "target workgroups out of range");
      c->policy.target_workgroups = (int32_t)value;
      return KVC_OK;
    case KVC_OPT_MAX_SPLITS:
      if (value < 1 || value > KVC_MAX_SPLITS) return fail(c, KVC_ERR_ARG, "max splits must be in [1, 64]");
      c->policy.max_splits = (int32_t)value;
      return KVC_OK;
    case KVC_OPT_PROFILE:
      if (c->metadata_only && value) return fail(c, KVC_ERR_STATE, "metadata-only context has no kernels");
      c->profile = value != 0;
      return KVC_OK;
    case KVC_OPT_DEFER_EVICTION:
      if (value != 0 && value != 1) return fail(c, KVC_ERR_ARG, "defer eviction is 0 or 1");
      c->alloc.set_defer_eviction(value != 0);
      return KVC_OK;
    case KVC_OPT_QUERY_TILE:
      if (value != 0 && value != 16 && value != 32) return fail(c, KVC_ERR_ARG, "query tile is 0, 16 or 32");
      c->policy.query_tile = (int32_t)value;
      return KVC_OK;
    case KVC_OPT_FUSED_APPEND:
      if (value != 0 && value != 1) return fail(c, KVC_ERR_ARG, "fused append is 0 or 1");
      if (!value && deferred_pending(c)) return fail(c, KVC_ERR_STATE, "a deferred append is pending");
      c->policy.fused = value != 0;
      return KVC_OK;
    default:
      return fail(c, KVC_ERR_ARG, "unknown option");
  }
}

kvc_status kvc_get_option(const kvc_ctx* c, int32_t option, int64_t* value) {
  if (!c || !value) return KVC_ERR_ARG;
  switch (option) {
    case KVC_OPT_TARGET_WORKGROUPS: *value = c->policy.target_workgroups; return KVC_OK;
    case KVC_OPT_MAX_SPLITS: *value = c->policy.max_splits; return KVC_OK;
    case KVC_OPT_PROFILE: *value = c->profile ? 1 : 0; return KVC_OK;
    case KVC_OPT_DEFER_EVICTION: *value = c->alloc.defer_eviction() ? 1 : 0; return KVC_OK;
    case KVC_OPT_QUERY_TILE: *value = c->policy.query_tile; return KVC_OK;
    case KVC_OPT_FUSED_APPEND: *value = c->policy.fused ? 1 : 0; return KVC_OK;
    default: return KVC_ERR_ARG;
  }
}

kvc_status kvc_profile_read(kvc_ctx* c, int32_t kernel, double* total_ms, int64_t* launches, int32_t reset) {
  if (!c || kernel < 0 || kernel >= KVC_NUM_KERNELS) return KVC_ERR_ARG;
  for (auto& ev : c->pending[kernel]) {
    hipError_t e = hipEventSynchronize(ev.stop);
    if (e != hipSuccess) return hip_fail(c, e, "profile event");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev.start, ev.stop);
    if (e != hipSuccess) return hip_fail(c, e, "profile elapsed");
    c->prof_ms[kernel] += ms;
    c->prof_n[kernel] += 1;
    c->spare.push_back(ev.start);
    c->spare.push_back(ev.stop);
  }
  c->pending[kernel].clear();
  if (total_ms) *total_ms = c->prof_ms[kernel];
  if (launches) *launches = c->prof_n[kernel];
  if (reset) {
    c->prof_ms[kernel] = 0;
    c->prof_n[kernel] = 0;
  }
  return KVC_OK;
}

const char* kvc_last_error(const kvc_ctx* c) { return c ? c->err.c_str() : "null context"; }

}  // extern "C"
