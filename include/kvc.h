/*
 * kvc.h - two-stream paged KV-cache prefill attention for streaming 3-D
 * reconstruction, native to AMD Instinct MI355X (gfx950).
 *
 * Sources are five web pages on the lingbot-map paged KV cache, cited by tag
 * and section:
 *   [p1] "How FlashInfer KV Cache Attention Accelerates Streaming 3D
 *        Reconstruction Over SDPA"
 *   [p2] "How LingBot-Map Uses FlashInfer KV Cache for Streaming 3D
 *        Reconstruction"
 *   [p3] "How FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback
 *        in Streaming Inference"
 *   [p4] "FlashInfer Backend in LingBot-Map: Accelerating Streaming Inference
 *        with Paged KV Cache"
 *   [p5] "How Paged KV Cache Attention Achieves Stable Inference in
 *        Ling-Bot-Map"
 *
 * What the library computes.  Each transformer block owns a page pool
 * [max_num_pages, 2, page_size, H, D] of bf16 in NHD order, dimension 1 being
 * 0 = K and 1 = V ([p1] §Paged KV Cache Memory Layout; [p5] §Core
 * Implementation Mechanics).  Patch page IDs are [0, max_patch_pages), special
 * page IDs [max_patch_pages, max_num_pages) ([p2] §Patch Stream and Special
 * Stream).  Each frame's patch tokens fill one recyclable patch page; its
 * special tokens pack continuously into an append-only special stream
 * ([p3] §Two-Stream Design).  The frame's queries then attend, without a mask,
 * over the visible page table scale -> live window -> specials, the last page
 * holding last_page_len valid tokens ([p2] §Page Table Planning and Reuse):
 *     o = softmax(q K^T / sqrt(D)) V   over every valid visible token.
 * One plan is built per frame step and reused by every block ([p3] §Plan-Run
 * Execution Workflow).
 *
 * Conventions.
 *   - Every call returns kvc_status: KVC_OK (0) or a negative error code.  On
 *     error kvc_last_error() describes it and host state is unchanged, except
 *     for KVC_ERR_HIP where a device call failed after host state changed.
 *   - Device pointers are HIP device addresses; "host" pointers are ordinary
 *     process memory.  The caller owns every buffer it passes; the library
 *     never allocates or frees device memory, so the device footprint is fixed
 *     when the caller allocates the pools and workspace ([p5] FAQ on the
 *     sliding window: memory does not grow with stream length).
 *   - Device work is enqueued on the caller's HIP stream (kvc_stream_t is a
 *     hipStream_t; NULL is the null stream).  Use one stream per context.
 *   - A context is not thread-safe.
 *
 * Per frame step, the calls must come in this order ([p1] §FlashInferAttention
 * Forward Pass: append, evict, then attention with the shared plan):
 *   1. kvc_append_frame(s, block 0, ...) for every stream s that advances
 *      (allocates its pages);
 *   2. kvc_evict(s) for those streams;
 *   3. kvc_plan() once (plans the streams of step 1, ascending stream index);
 *   4. kvc_run(block 0, ...);
 *   5. for every block b >= 1: kvc_append_frame(s, b, ...) for every planned
 *      stream, then kvc_run(b, ...).
 * Out-of-order calls return KVC_ERR_STATE.  kvc_plan ends a step: the first
 * kvc_append_frame(s, 0) after it starts the next one.  A step that runs no
 * attention (streaming ahead) is still closed by kvc_plan, which then only
 * costs the host build and one small copy.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 8

typedef struct kvc_ctx kvc_ctx;
typedef void* kvc_stream_t;   /* hipStream_t */
typedef int32_t kvc_status;

enum {
  KVC_OK = 0,
  KVC_ERR_ARG = -1,             /* bad argument (null, out of range, wrong size) */
  KVC_ERR_STATE = -2,           /* call out of the per-step order */
  KVC_ERR_POOL_EXHAUSTED = -3,  /* no free patch page, or the special pool is full ([p2] §Patch Stream and Special Stream) */
  KVC_ERR_CAPACITY = -4,        /* configuration cannot hold the steady state */
  KVC_ERR_HIP = -5,             /* a HIP runtime call failed */
  KVC_ERR_UNSUPPORTED = -6,     /* shape outside what the kernels are built for */
  KVC_ERR_HOST_ALLOC = -7       /* the library could not allocate host memory for a context */
};

/* Sizing and shape of one cache ([p2] §Initializing the Cache Manager;
 * [p5] §Initializing the Cache Manager).  All fields are required. */
typedef struct kvc_config {
  int32_t num_blocks;          /* transformer blocks, one pool each, >= 1 */
  int32_t num_heads;           /* H: query and KV heads, >= 1 */
  int32_t head_dim;            /* D: 32, 64 or 128 */
  int32_t tokens_per_frame;    /* T = patch tokens P + special tokens n_s, >= 1 */
  int32_t num_special_tokens;  /* n_s, 0 <= n_s < T, n_s <= 64 */
  int32_t special_row_offset;  /* row of a frame's first special token in its [T] rows;
                                  patch rows are the others in order (P means specials last) */
  int32_t page_size;           /* tokens per page, >= P; P gives unpadded patch pages and larger
                                  values zero-padded ones ([p1] §Efficient Attention Masking and Padding) */
  int32_t scale_frames;        /* S: first S frames kept permanently ([p2] §Scale Frames vs Sliding Window) */
  int32_t sliding_window;      /* W >= 1: most recent non-scale frames kept */
  int32_t num_streams;         /* independent frame streams sharing the pools, >= 1 */
  int32_t max_patch_pages;     /* >= num_streams * (S + W + 1) */
  int32_t max_special_pages;   /* special pages shared by all streams, >= 0 */
  int32_t max_frames_per_step; /* most frames one stream appends in one step, 1..64: above 1 for the
                                  multi-frame scale phase ([p2] §Frame Processing Loop) */
  int32_t dtype;               /* element type of the pools and of every k, v, q, o buffer:
                                  KVC_DTYPE_BF16 (0) or KVC_DTYPE_F16 (1), the two 16-bit types the
                                  paged kernels take natively ([p3] §Precision and Hardware
                                  Utilization), or KVC_DTYPE_F32 (2), the full-precision pool ([p3]
                                  FAQ on fp32 precision; [p4] §Memory Management and Debugging);
                                  below, "bf16" reads as this type */
} kvc_config;

/* Element types (kvc_config.dtype).  With the 16-bit types arithmetic is
   MFMA on the 16-bit values with float32 accumulation and softmax, and the
   probabilities are rounded to the element type for the P.V product.  With
   float32, products, sums and the softmax are float32 throughout (float32
   MFMA, probabilities not rounded), every element takes 4 bytes, and
   attention runs without KV splits. */
enum { KVC_DTYPE_BF16 = 0, KVC_DTYPE_F16 = 1, KVC_DTYPE_F32 = 2 };

/* [p3] §Inspecting Cache Statistics, plus the special-page counters. */
typedef struct kvc_stats {
  int64_t frame_count;         /* frames appended to this stream since create/reset */
  int64_t special_tokens;      /* special tokens held by this stream */
  int32_t scale_pages;         /* scale patch pages of this stream */
  int32_t live_pages;          /* live-window patch pages of this stream */
  int32_t free_pages;          /* free patch pages (shared by all streams) */
  int32_t special_pages;       /* special pages of this stream */
  int32_t free_special_pages;  /* free special pages (shared) */
  int32_t reserved;
} kvc_stats;

/* Tunables for kvc_set_option / kvc_get_option. */
enum {
  KVC_OPT_TARGET_WORKGROUPS = 1, /* attention work-groups the planner fills per run without exceeding it
                                    (default: the device's compute-unit count, one resident work-group
                                    each; the 16-row kernel at head_dim 64 holds two per CU and fills
                                    twice this) */
  KVC_OPT_MAX_SPLITS = 2,        /* cap on KV splits per stream; 1 disables split-KV (default 64, the maximum) */
  KVC_OPT_PROFILE = 3,           /* 1: time every attention/merge/append/rope launch with HIP events */
  KVC_OPT_DEFER_EVICTION = 4,    /* 1: hold evicted window pages back until the stream's next frame,
                                    so that kvc_rollback can undo the latest frame (default 0) */
  KVC_OPT_QUERY_TILE = 5,        /* query rows per MFMA tile of the 16-bit attention kernel at head_dim 64:
                                    0 = the planner's choice (default), 16 or 32 = that kernel always.
                                    head_dim 32 has only the 32-row kernel, 128 only the 16-row one and
                                    float32 pools their own: there the setting is ignored */
  KVC_OPT_FUSED_APPEND = 6       /* 1: plans from the next kvc_plan on are built for kvc_run_append (the
                                    step's own rows form work units of their own); an append with
                                    k = v = NULL then defers its copy to that block's kvc_run_append
                                    (default 0; 0 is refused while a deferred append is pending) */
};

/* Kernels for kvc_profile_read. */
enum { KVC_KERNEL_ATTENTION = 0, KVC_KERNEL_MERGE = 1, KVC_KERNEL_APPEND = 2, KVC_KERNEL_ROPE = 3 };
#define KVC_NUM_KERNELS 4

int32_t kvc_abi_version(void);
const char* kvc_status_string(kvc_status status);

/* Bytes of ONE block's pool: max_num_pages * 2 * page_size * H * D * 2, where
 * max_num_pages = max_patch_pages + max_special_pages ([p2] §Physical Memory
 * Layout).  Returns 0 for an invalid configuration. */
size_t kvc_pool_bytes(const kvc_config* cfg);

/* Bytes of device workspace the caller allocates for kvc_create: two plan
 * buffers, the split-KV partial outputs (normalised bf16 outputs and float32
 * log-sum-exps) sized for the maximum split count, and the rotated query rows
 * of kvc_run_rope.  Returns 0 for an invalid configuration. */
size_t kvc_workspace_bytes(const kvc_config* cfg);

/* Bytes of pinned (page-locked) host staging for the per-step plan upload,
 * double-buffered.  The caller allocates it with hipHostMalloc or an
 * equivalent pinned allocator.  Returns 0 for an invalid configuration. */
size_t kvc_staging_bytes(const kvc_config* cfg);

/* Create a context on the current HIP device.
 *   cfg:        configuration, copied.
 *   pools:      host array of num_blocks device pointers, each to
 *               kvc_pool_bytes(cfg) bytes, 16-byte aligned; zero-filled here
 *               (synchronously) so pad slots are defined.
 *   workspace:  device pointer to kvc_workspace_bytes(cfg) bytes, 256-byte
 *               aligned.
 *   staging:    pinned host pointer to kvc_staging_bytes(cfg) bytes.
 *   free_patch_order / free_special_order: optional host arrays giving the
 *               initial order of the free lists (permutations of
 *               [0, max_patch_pages) and [max_patch_pages, max_num_pages));
 *               NULL means ascending.  Pages are taken from the front and
 *               freed to the back ([p1] §Two-Stream Design for Token Types:
 *               deques).
 *   out:        receives the context.
 * Errors: KVC_ERR_ARG, KVC_ERR_CAPACITY (max_patch_pages too small),
 * KVC_ERR_UNSUPPORTED (head_dim, or a shape the kernels do not cover),
 * KVC_ERR_HOST_ALLOC, KVC_ERR_HIP. */
kvc_status kvc_create(const kvc_config* cfg, void* const* pools, void* workspace, void* staging,
                      const int32_t* free_patch_order, const int32_t* free_special_order,
                      kvc_ctx** out);

/* Create a context that keeps only the page bookkeeping and planning (no
 * device buffers, no HIP calls).  kvc_append_frame takes k = v = NULL and
 * only allocates; kvc_plan builds the host plan only; kvc_run returns
 * KVC_ERR_STATE.  Used to replay or inspect plans without a GPU. */
kvc_status kvc_create_metadata_only(const kvc_config* cfg, const int32_t* free_patch_order,
                                    const int32_t* free_special_order, kvc_ctx** out);

kvc_status kvc_destroy(kvc_ctx* ctx);

/* [p5] §Resetting for New Sequences: clear page lists and counters and keep
 * the buffers (pool contents are left as they are; only valid visible slots
 * are ever read).  Every per-step state is cleared too: the step in progress
 * is dropped, kvc_get_plan has no plan, and the next call must be a block-0
 * append. */
kvc_status kvc_reset(kvc_ctx* ctx);

/* Write one frame's K and V for one block ([p5] §Frame Appending Without
 * Dispatch Overhead; [p3] §Two-Stream Design).
 *   k, v: device [T, H, D] bf16, NHD, contiguous, 16-byte aligned.
 * At block 0 this also allocates the frame: one patch page from the free list
 * (a scale page while the stream has fewer than S, else a live-window page)
 * and the next n_s slots of the stream's special stream, taking a new special
 * page whenever the tail page is full.  Blocks >= 1 reuse that page and those
 * slots.  One kernel launch writes the patch rows to slots [0, P) of the page
 * and each special row to its slot; pad slots are never written.
 * With KVC_OPT_FUSED_APPEND on a device context, k = v = NULL does the
 * bookkeeping (and at block 0 the allocation) without the copy, which the
 * block's kvc_run_append then makes.
 * Errors: KVC_ERR_ARG, KVC_ERR_STATE (block >= 1 before block 0 of the step,
 * a block appended twice in one step, or a new step while an append of the
 * last one is still deferred), KVC_ERR_POOL_EXHAUSTED (block 0 only; nothing
 * changes), KVC_ERR_HIP. */
kvc_status kvc_append_frame(kvc_ctx* ctx, int32_t stream, int32_t block, const void* k, const void* v,
                            kvc_stream_t hip_stream);

/* Several frames of one stream in one step: the scale phase, where the first
 * frames are processed together and every frame's K/V is appended ([p2]
 * §Frame Processing Loop, num_frames > 1).
 *   k, v: device [num_frames, T, H, D] bf16, contiguous, 16-byte aligned.
 *   num_frames: 1..max_frames_per_step; every block of the step passes the
 *   same count.
 * At block 0 the frames are allocated in order, exactly as num_frames calls
 * of kvc_append_frame would (all or none: on KVC_ERR_POOL_EXHAUSTED nothing
 * changes).  The step's queries are then the num_frames * T rows of those
 * frames, and they attend to every visible token, the step's own frames
 * included.  kvc_append_frame is this call with num_frames = 1.
 * Errors: as kvc_append_frame, and KVC_ERR_ARG for a count outside
 * 1..max_frames_per_step or different from block 0's. */
kvc_status kvc_append_frames(kvc_ctx* ctx, int32_t stream, int32_t block, const void* k, const void* v,
                             int32_t num_frames, kvc_stream_t hip_stream);

/* kvc_append_frames with the rotary position embedding applied to K on its
 * way into the pool ([p2] "How LingBot-Map Uses FlashInfer KV Cache for
 * Streaming 3D Reconstruction" §3D RoPE Position Encoding and its FAQ on
 * temporal information: positions are baked into q and k before the cache,
 * so attention needs no position lookup).  The pages give no frequencies, so
 * the angles are the caller's:
 *   rope_cos, rope_sin: device float32 [num_frames * T, D/2], contiguous,
 *   16-byte aligned; entry (t, i) is the cosine (sine) of the angle by which
 *   elements (2i, 2i+1) of every head of k row t turn:
 *     (a, b) -> (a cos - b sin, a sin + b cos).
 * The rotation is computed in float64 (both products are exact there) and
 * rounded once to the element type, nearest even.  V is stored as it is.
 * Nothing is written to k, v or the tables.  Errors: as kvc_append_frames,
 * and KVC_ERR_ARG for a null or misaligned table (a metadata-only context
 * takes none). */
kvc_status kvc_append_frames_rope(kvc_ctx* ctx, int32_t stream, int32_t block, const void* k, const void* v,
                                  int32_t num_frames, const float* rope_cos, const float* rope_sin,
                                  kvc_stream_t hip_stream);

/* [p5] §Sliding-Window Eviction Strategy: move the oldest live-window pages
 * beyond the window back to the free list (host metadata only; scale pages
 * are kept).  Idempotent within a step.  With KVC_OPT_DEFER_EVICTION the
 * pages leave the visible table but are held back (their contents intact)
 * until the stream appends its next frame. */
kvc_status kvc_evict(kvc_ctx* ctx, int32_t stream);

/* Deferred eviction for frame rollback, as key-frame selection needs ([p2]
 * §Scale Frames vs Sliding Window; [p4] §Summary): undo the stream's most
 * recent frame.  Its patch page and the special pages it opened return to
 * the front of the free lists, its special tokens are dropped, and window
 * pages held back by the last eviction return to the front of the window
 * until it is full; no device memory is touched.  The visible table is then
 * the one before that frame, and the next frame reuses the freed page.
 * Call between steps (after kvc_plan); the step's plan can no longer be run.
 * Errors: KVC_ERR_ARG, KVC_ERR_STATE (deferred eviction off, mid-step, or no
 * frame to undo: only the latest frame, once per append). */
kvc_status kvc_rollback(kvc_ctx* ctx, int32_t stream);

/* Build the step's plan ([p3] §Plan-Run Execution Workflow): for each stream
 * that appended block 0 this step, in ascending order, the visible page table
 * (scale -> live window -> specials, [p2] §Page Table Planning and Reuse),
 * the last page length ([p5] §Kernel Dispatch and Sequence Lengths), the
 * query row ranges and the split-KV work list; then one asynchronous copy of
 * the plan from pinned staging to the workspace on hip_stream.
 * Errors: KVC_ERR_STATE (no stream appended, or already planned this step),
 * KVC_ERR_CAPACITY (a planned stream holds more than scale_frames +
 * sliding_window patch pages, i.e. kvc_evict was skipped: the plan would not
 * fit the plan buffer; or a planned stream sees more than 2^21 tokens, beyond
 * 64 KV splits of 512 work units of 64 slots; nothing changes), KVC_ERR_HIP. */
kvc_status kvc_plan(kvc_ctx* ctx, kvc_stream_t hip_stream);

/* Paged attention for one block with the step's plan ([p2] §Attention Kernel
 * Execution):
 *   q: device [R, H, D] bf16, R = T * (frames appended this step, summed over
 *      the planned streams), rows in plan order (stream i's frames at rows
 *      [qo_indptr[i], qo_indptr[i+1]), frame by frame).
 *   o: device [R, H, D] bf16, written; must not overlap q.
 * Each stream's queries attend only to its own visible tokens.  Launches the
 * attention kernel and, when a stream's KV is split, the merge kernel.
 * Every run and plan of one context uses the same workspace (plan buffers and
 * split partials), so they must execute in call order on the device: issue
 * them on one HIP stream, or order the streams with events.  Runs of different
 * contexts are independent.
 * Errors: KVC_ERR_ARG, KVC_ERR_STATE (not planned, or a planned stream has
 * not appended this block), KVC_ERR_HIP. */
kvc_status kvc_run(kvc_ctx* ctx, int32_t block, const void* q, void* o, kvc_stream_t hip_stream);

/* The append of this step's frames for one block and its attention, fused
 * ([p5] "How Paged KV Cache Attention Achieves Stable Inference in
 * Ling-Bot-Map" §Frame Appending Without Dispatch Overhead; [p2] "How
 * LingBot-Map Uses FlashInfer KV Cache for Streaming 3D Reconstruction"
 * §Attention Kernel Execution): the result and the pool afterwards are those
 * of kvc_append_frames of every planned stream followed by kvc_run.  Needs a
 * plan built with KVC_OPT_FUSED_APPEND; at block 0 the planned streams have
 * appended with k = v = NULL (deferred), at blocks >= 1 they may have or not.
 *   k, v: host arrays of num_streams device pointers, indexed by stream id;
 *         entry s of a planned stream is its [num_frames, T, H, D] rows as
 *         kvc_append_frames takes them (other entries are not read).  They
 *         must stay unchanged until the launches on hip_stream complete.
 *   q, o: as kvc_run.
 * With the 32-row kernel (head_dim 32, 64), a split plan and at most 4
 * planned streams, the attention kernel reads the step's own rows straight
 * from k and v (the plan gives them work units of their own) and the merge
 * launch also copies them into the pool: two launches instead of the
 * append's, the attention's and the merge's.  Otherwise the appends are
 * launched, then the run, with the same result.
 * Errors: KVC_ERR_ARG, KVC_ERR_STATE (not planned; the plan built without
 * the option; a planned stream already appended this block with data, or
 * has not appended block 0), KVC_ERR_HIP. */
kvc_status kvc_run_append(kvc_ctx* ctx, int32_t block, const void* const* k, const void* const* v, const void* q,
                          void* o, kvc_stream_t hip_stream);

/* kvc_run with the rotary position embedding applied to the queries first
 * (the same section as kvc_append_frames_rope, the same arithmetic):
 *   rope_cos, rope_sin: device float32 [R, D/2], contiguous, 16-byte aligned,
 *   rows in q's order.
 * One pass writes the rotated rows into the workspace (q itself is not
 * changed), then attention runs on them as kvc_run does.  Errors: as kvc_run,
 * and KVC_ERR_ARG for a null or misaligned table. */
kvc_status kvc_run_rope(kvc_ctx* ctx, int32_t block, const void* q, const float* rope_cos,
                        const float* rope_sin, void* o, kvc_stream_t hip_stream);

/* Size of the static device scratch behind kvc_run_no_alloc, per device. */
#define KVC_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory while they run attention:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  kvc_run with the split-KV partial outputs (the per-split
 * normalised outputs and log-sum-exps that the attention kernel writes and the
 * merge kernel reads back) kept in a static device array of
 * KVC_NO_ALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends, instead of in the context's workspace.  Arguments,
 * call order and results are those of kvc_run; the plan still comes from the
 * context's workspace.  Nothing is allocated: no hipMalloc, no hipFree, no
 * allocating library call (the device address of the array is looked up once
 * per device, on the first call made with that device current).
 * Every call on one device shares that device's array, and it keeps the last
 * call's contents (nothing in it needs to start at zero: every partial is
 * written before it is read).  Calls that overlap on one device (on different
 * streams, or from different contexts at the same time) race on the array;
 * calls issued in order on one stream do not.
 * Errors: as kvc_run, and KVC_ERR_CAPACITY when the step's plan needs more
 * partial-output space than the array holds (splits x heads x query tiles of
 * the configuration); nothing is launched then. */
kvc_status kvc_run_no_alloc(kvc_ctx* ctx, int32_t block, const void* q, void* o, kvc_stream_t hip_stream);

/* Copy the current plan to host arrays (for bit-exact checks).
 *   planned_streams[capacity_streams], kv_indptr[capacity_streams + 1],
 *   last_page_len[capacity_streams], n_patch_pages[capacity_streams],
 *   qo_indptr[capacity_streams + 1], n_splits[capacity_streams]:
 *   per planned stream; kv_indices[capacity_indices]: concatenated tables.
 *   Any array pointer may be NULL.  num_planned / num_indices receive the
 *   sizes.  Errors: KVC_ERR_STATE (no plan), KVC_ERR_ARG (capacity short). */
kvc_status kvc_get_plan(const kvc_ctx* ctx, int32_t* planned_streams, int32_t* kv_indptr,
                        int32_t* kv_indices, int32_t* last_page_len, int32_t* n_patch_pages,
                        int32_t* qo_indptr, int32_t* n_splits, int32_t capacity_streams,
                        int32_t capacity_indices, int32_t* num_planned, int32_t* num_indices);

/* Shape of the current plan's attention launch (for tests and tuning):
 *   work_items: attention work-groups, (stream, head, KV split, query group);
 *   group_rows: most query rows one work-group covers.  The 32-row kernel
 *               (head_dim 32, and 64 unless the plan takes the 16-row one):
 *               4 waves x 2 tiles x 32 rows = 256, plus 16 when the launch
 *               lets a group carry a tail of up to 16 rows shared by the
 *               waves (272); the 16-row kernel (head_dim 128, and 64 where
 *               the planner or KVC_OPT_QUERY_TILE picks it): 8 tiles x 16
 *               rows = 128, or 144 with a ninth tile shared by the waves
 *               (head_dim 128 only); float32 pools: 16.
 * Either pointer may be NULL.  Errors: KVC_ERR_ARG, KVC_ERR_STATE (no plan). */
kvc_status kvc_get_plan_shape(const kvc_ctx* ctx, int32_t* work_items, int32_t* group_rows);

/* Copy the current plan's device image (the int32 buffer that kvc_plan
 * uploads and the kernels read; layout in kvc_plan_layout.h of the sources)
 * to buf, for host-side checks.  capacity: ints available in buf (buf may be
 * NULL to query the size); n_ints receives the image's size.
 * Errors: KVC_ERR_ARG (capacity short), KVC_ERR_STATE (no plan). */
kvc_status kvc_get_plan_image(const kvc_ctx* ctx, int32_t* buf, int32_t capacity, int32_t* n_ints);

/* Copy the split partial results that the latest kvc_run wrote (for tests
 * of the split-KV decomposition; [p5] "How Paged KV Cache Attention Achieves
 * Stable Inference in Ling-Bot-Map" §Kernel Dispatch and Sequence Lengths:
 * the splits of a row must combine to the exact softmax over its valid
 * tokens).  Waits for hip_stream, then copies device to host:
 *   lse: float [KVC_MAX_SPLITS][H][tiles][32], the base-2 log-sum-exp of the
 *        scores (q.k / sqrt(D)) of each query row over the split's tokens;
 *   o:   element type [KVC_MAX_SPLITS][H][tiles][D/32][4][64][4], the split's
 *        normalised output, element (d, row) at [d/32][(d%32)/8]
 *        [32 ((d%8)/4) + row][d%4] of its 32-row tile,
 * with tiles = num_streams * ceil(max_frames_per_step * tokens_per_frame / 32)
 * and a stream's tiles from its first (the plan's query tiles in order).
 * Only the splits and tiles of split streams in the current plan hold
 * values.  Either pointer may be NULL; n_lse / n_o receive the element counts.
 * Errors: KVC_ERR_ARG (capacity short), KVC_ERR_STATE (no plan), KVC_ERR_HIP. */
kvc_status kvc_get_split_partials(const kvc_ctx* ctx, float* lse, int64_t capacity_lse, uint16_t* o,
                                  int64_t capacity_o, int64_t* n_lse, int64_t* n_o, kvc_stream_t hip_stream);

/* [p3] §Inspecting Cache Statistics for one stream. */
kvc_status kvc_get_stats(const kvc_ctx* ctx, int32_t stream, kvc_stats* out);

kvc_status kvc_set_option(kvc_ctx* ctx, int32_t option, int64_t value);
kvc_status kvc_get_option(const kvc_ctx* ctx, int32_t option, int64_t* value);

/* Launch timing collected while KVC_OPT_PROFILE is 1: total milliseconds and
 * number of launches of one kernel (KVC_KERNEL_*), measured with HIP events
 * recorded around each launch on its stream.  Synchronizes with the recorded
 * events.  reset != 0 clears the counters afterwards. */
kvc_status kvc_profile_read(kvc_ctx* ctx, int32_t kernel, double* total_ms, int64_t* launches, int32_t reset);

/* Description of the last error on this context (empty when none). */
const char* kvc_last_error(const kvc_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
