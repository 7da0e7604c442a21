"""C-ABI library checks that need no GPU: it loads, exports every symbol that
include/kvc.h declares, and its host allocator and planner (driven through a
metadata-only context) reproduce the oracle's page tables, last-page lengths
and cache statistics bit for bit on every step of every workload; error paths
and the per-step call order are enforced."""
import ctypes
import os
import re

import numpy as np
import pytest

import kvc_synth as syn
import paged_kv_cache_kvc_amd as kvc
from oracle import kvc_oracle as ko

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = kvc.load_library()
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
        assert n in kvc.SIGNATURES, n
    assert set(kvc.SIGNATURES) == set(names)
    assert lib.kvc_abi_version() == kvc.ABI_VERSION == 8


def cfg_of(wl: syn.Workload):
    return kvc.make_config(wl.num_blocks, wl.num_heads, wl.head_dim, wl.tokens_per_frame, wl.num_special_tokens,
                           page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                           num_streams=wl.num_streams, max_patch_pages=wl.max_patch_pages,
                           max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset)


def ocfg_of(wl: syn.Workload):
    return ko.OracleConfig(num_heads=wl.num_heads, head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame,
                           num_special_tokens=wl.num_special_tokens, page_size=wl.page_size,
                           scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                           max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages,
                           num_streams=wl.num_streams, special_row_offset=wl.special_row_offset)


def free_orders(wl):
    if not wl.shuffle_free_lists:
        return None, None
    return (syn.free_list_order(wl.seed, wl.max_patch_pages, 0, 0),
            syn.free_list_order(wl.seed, wl.max_special_pages, wl.max_patch_pages, 1))


def compare_plans(ours, ref, active):
    assert list(ours["planned"]) == list(active)
    for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr"):
        assert np.array_equal(ours[k], ref[k]), k


@pytest.mark.parametrize("name", ["tiny", "base", "r518", "long", "frag"])
def test_metadata_replay_matches_oracle_every_step(name):
    wl = syn.WORKLOADS[name]
    po, so = free_orders(wl)
    cache = kvc.PagedKVCache(cfg_of(wl), metadata_only=True, free_patch_order=po, free_special_order=so)
    ref = ko.AllocatorReplay(ocfg_of(wl), po, so)
    total = max(wl.frames)
    for step in range(total):
        active = [s for s in range(wl.num_streams) if step >= syn.stream_join_step(wl, s)]
        for s in active:
            cache.append_frame(0, stream_id=s)
            ref.append_frame(s)
        for s in active:
            cache.evict_frames(s)
            ref.evict_frames(s)
        cache.plan()
        compare_plans(cache.get_plan(), ref.plan(active), active)
        if step % 50 == 0 or step == total - 1:
            for s in active:
                ours = cache.get_cache_stats(s)
                theirs = ref.get_cache_stats(s)
                assert {k: ours[k] for k in theirs} == theirs
    # split count never exceeds the KV tiles of a stream
    p = cache.get_plan()
    assert np.all(p["n_splits"] >= 1) and np.all(p["n_splits"] <= kvc.MAX_SPLITS)


@pytest.mark.parametrize("name", ["no_specials", "max_specials", "one_token", "steps_of_64"])
def test_metadata_replay_degenerate_shapes(name):
    """Page tables and counters of the degenerate shapes against the oracle at
    every step (the 64-frame shape appends its first 64 frames in one step)."""
    from tests.stream_harness import cfg_args, edge_workloads
    wl = edge_workloads()[name]
    multi = 64 if name == "steps_of_64" else 1
    cache = kvc.PagedKVCache(kvc.make_config(**cfg_args(wl, 1), max_frames_per_step=multi), metadata_only=True)
    ref = ko.AllocatorReplay(ocfg_of(wl))
    done = 0
    while done < max(wl.frames):
        nf = multi if done == 0 else 1
        if nf > 1:
            cache.append_frames(0, num_frames=nf)
        else:
            cache.append_frame(0)
        for _ in range(nf):
            ref.append_frame(0)
        cache.evict_frames(0)
        ref.evict_frames(0)
        cache.plan()
        compare_plans(cache.get_plan(), ref.plan([0], frames=[nf]), [0])
        st, rs = cache.get_cache_stats(0), ref.get_cache_stats(0)
        assert {k: st[k] for k in rs} == rs
        done += nf


def test_worked_example_through_abi():
    cfg = kvc.make_config(1, 16, 64, 262, 6, scale_frames=8, sliding_window=64, max_patch_pages=88,
                          max_total_frames=200)
    cache = kvc.PagedKVCache(cfg, metadata_only=True)
    for _ in range(42):
        cache.append_frame(0)
        cache.evict_frames()
        cache.plan()
    st = cache.get_cache_stats()
    assert {k: st[k] for k in ("frame_count", "scale_pages", "live_pages", "free_pages", "special_tokens")} == \
        {"frame_count": 42, "scale_pages": 8, "live_pages": 34, "free_pages": 46, "special_tokens": 252}


def tiny_cache(**kw):
    wl = syn.WORKLOADS["tiny"]
    c = cfg_of(wl)
    for k, v in kw.items():
        setattr(c, k, v)
    return kvc.PagedKVCache(c, metadata_only=True)


def test_call_order_is_enforced():
    c = tiny_cache(num_blocks=3)
    with pytest.raises(kvc.KvcError) as e:
        c.plan()                                   # nothing appended
    assert e.value.status == kvc.KVC_ERR_STATE
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(1)                          # block 1 before block 0
    assert e.value.status == kvc.KVC_ERR_STATE
    c.append_frame(0)
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(0)                          # block 0 twice in one step
    assert e.value.status == kvc.KVC_ERR_STATE
    c.append_frame(2)
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(2)                          # block appended twice in one step
    assert e.value.status == kvc.KVC_ERR_STATE
    c.evict_frames()
    c.plan()
    with pytest.raises(kvc.KvcError) as e:
        c.plan()                                   # second plan in a step
    assert e.value.status == kvc.KVC_ERR_STATE
    c.append_frame(1)
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(1)                          # block appended twice
    assert e.value.status == kvc.KVC_ERR_STATE
    # run is refused on a metadata-only context
    lib = kvc.load_library()
    assert lib.kvc_run(c._ctx, 0, 16, 32, None) == kvc.KVC_ERR_STATE
    # next step starts with block 0
    c.append_frame(0)
    assert c.get_cache_stats()["frame_count"] == 2


def test_bad_arguments_and_capacity():
    lib = kvc.load_library()
    wl = syn.WORKLOADS["tiny"]
    good = cfg_of(wl)
    assert lib.kvc_pool_bytes(ctypes.byref(good)) == (6 + 5) * 2 * 16 * 2 * 32 * 2
    bad = cfg_of(wl)
    bad.head_dim = 48
    ctx = ctypes.c_void_p()
    assert lib.kvc_create_metadata_only(ctypes.byref(bad), None, None, ctypes.byref(ctx)) == kvc.KVC_ERR_UNSUPPORTED
    assert lib.kvc_pool_bytes(ctypes.byref(bad)) == 0
    small = cfg_of(wl)
    small.max_patch_pages = wl.scale_frames + wl.sliding_window      # no room for the appended frame
    assert lib.kvc_create_metadata_only(ctypes.byref(small), None, None, ctypes.byref(ctx)) == kvc.KVC_ERR_CAPACITY
    dt = cfg_of(wl)
    dt.dtype = 3                                                      # none of bf16, f16, f32
    assert lib.kvc_create_metadata_only(ctypes.byref(dt), None, None, ctypes.byref(ctx)) == kvc.KVC_ERR_UNSUPPORTED
    assert lib.kvc_pool_bytes(ctypes.byref(dt)) == 0
    dt.dtype = kvc.KVC_DTYPE_F16                                      # same sizes as bf16
    assert lib.kvc_pool_bytes(ctypes.byref(dt)) == lib.kvc_pool_bytes(ctypes.byref(good))
    dt.dtype = kvc.KVC_DTYPE_F32                                      # 4-byte elements
    assert lib.kvc_pool_bytes(ctypes.byref(dt)) == 2 * lib.kvc_pool_bytes(ctypes.byref(good))
    assert lib.kvc_workspace_bytes(ctypes.byref(dt)) > lib.kvc_workspace_bytes(ctypes.byref(good))
    with pytest.raises(kvc.KvcError):
        kvc.make_config(1, 2, 32, 22, dtype="fp8")
    pg = cfg_of(wl)
    pg.page_size = 15                                                 # < P
    assert lib.kvc_create_metadata_only(ctypes.byref(pg), None, None, ctypes.byref(ctx)) == kvc.KVC_ERR_ARG
    # free-list orders must be permutations
    dup = np.zeros(wl.max_patch_pages, np.int32)
    assert lib.kvc_create_metadata_only(ctypes.byref(good), dup.ctypes.data_as(kvc._PI32), None,
                                        ctypes.byref(ctx)) == kvc.KVC_ERR_ARG
    c = tiny_cache()
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(0, stream_id=1)
    assert e.value.status == kvc.KVC_ERR_ARG
    with pytest.raises(kvc.KvcError) as e:
        c.set_option(kvc.KVC_OPT_MAX_SPLITS, 65)
    assert e.value.status == kvc.KVC_ERR_ARG
    assert lib.kvc_create(ctypes.byref(good), None, None, None, None, None, ctypes.byref(ctx)) == kvc.KVC_ERR_ARG


def test_special_pool_exhaustion_at_predicted_frame_leaves_state():
    c = tiny_cache(max_special_pages=3)          # 48 slots = 8 frames of 6 specials
    for _ in range(8):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
    before = c.get_cache_stats()
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(0)
    assert e.value.status == kvc.KVC_ERR_POOL_EXHAUSTED
    assert c.get_cache_stats() == before


def test_patch_pool_exhaustion_without_eviction():
    c = tiny_cache()                             # 6 patch pages, never evicted
    for _ in range(6):
        c.append_frame(0)
        c.plan()
    with pytest.raises(kvc.KvcError) as e:
        c.append_frame(0)
    assert e.value.status == kvc.KVC_ERR_POOL_EXHAUSTED


def test_plan_without_eviction_is_refused_not_overrun():
    """A stream that keeps appending without kvc_evict holds more window pages
    than the plan buffer is sized for (scale_frames + sliding_window per
    stream).  kvc_plan must refuse that plan with KVC_ERR_CAPACITY before
    anything is copied, and leave the step open; evicting then lets the same
    step plan."""
    wl = syn.WORKLOADS["base"]
    cfg = kvc.make_config(1, wl.num_heads, wl.head_dim, wl.tokens_per_frame, wl.num_special_tokens,
                          page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                          max_patch_pages=4000, max_special_pages=60)
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    refused = None
    for f in range(2000):
        c.append_frame(0)
        try:
            c.plan()
        except kvc.KvcError as e:
            assert e.status == kvc.KVC_ERR_CAPACITY
            refused = f
            break
    assert refused is not None and refused > wl.scale_frames + wl.sliding_window
    # the step is still open: evicting and planning it succeeds
    with pytest.raises(kvc.KvcError) as e2:
        c.append_frame(0)
    assert e2.value.status == kvc.KVC_ERR_STATE
    c.evict_frames()
    c.plan()
    p = c.get_plan()
    assert p["n_patch_pages"][0] == wl.scale_frames + wl.sliding_window
    img = c.get_plan_image()
    assert img.size > 0


def test_reset_clears_every_per_step_state():
    """kvc_reset in the middle of a step drops the step: no plan is left, a
    block-1 append or a plan is out of order, and a multi-frame count of the
    dropped step does not constrain the next one."""
    base = syn.WORKLOADS["base"]
    cfg = kvc.make_config(2, 2, 32, base.tokens_per_frame, base.num_special_tokens, page_size=base.page_size,
                          scale_frames=2, sliding_window=4, max_patch_pages=2 + 4 + 8, max_special_pages=8,
                          max_frames_per_step=4)
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    c.append_frames(0, num_frames=3)
    c.reset()
    with pytest.raises(kvc.KvcError) as e:
        c.get_plan()
    assert e.value.status == kvc.KVC_ERR_STATE
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(1, num_frames=3)
    assert e.value.status == kvc.KVC_ERR_STATE
    with pytest.raises(kvc.KvcError) as e:
        c.plan()
    assert e.value.status == kvc.KVC_ERR_STATE
    c.append_frames(0, num_frames=2)
    c.append_frames(1, num_frames=2)
    c.evict_frames()
    c.plan()
    assert list(c.get_plan()["qo_indptr"]) == [0, 2 * base.tokens_per_frame]
    assert c.get_cache_stats()["frame_count"] == 2


def test_reset_replays_like_fresh():
    c = tiny_cache()
    plans = []
    for _ in range(10):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
        plans.append(c.get_plan())
    c.reset()
    for i in range(10):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
        p = c.get_plan()
        for k in plans[i]:
            assert np.array_equal(p[k], plans[i][k])


def test_split_policy_options():
    wl = syn.WORKLOADS["base"]
    c = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    for _ in range(200):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
    default = c.get_plan()["n_splits"][0]
    assert default > 1
    c.set_option(kvc.KVC_OPT_MAX_SPLITS, 1)
    c.append_frame(0)
    c.plan()
    assert c.get_plan()["n_splits"][0] == 1
    assert c.get_option(kvc.KVC_OPT_MAX_SPLITS) == 1


def _plan_at_measured_step(name):
    wl = syn.WORKLOADS[name]
    c = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    F = max(wl.frames)
    starts = [F - f for f in wl.frames]
    for t in range(F):
        act = [s for s in range(len(wl.frames)) if t >= starts[s]]
        for s in act:
            c.append_frame(0, stream_id=s)
        for s in act:
            c.evict_frames(stream_id=s)
        c.plan()
    return wl, c


def _units_and_qtiles(wl, p):
    P = wl.tokens_per_frame - wl.num_special_tokens
    ceil = lambda a, b: -(-a // b)
    units, qtiles = [], []
    for i in range(len(p["planned"])):
        n_pages = int(p["kv_indptr"][i + 1] - p["kv_indptr"][i])
        n_patch = int(p["n_patch_pages"][i])
        n_sp = n_pages - n_patch
        u = n_patch * ceil(P, 64)
        if n_sp:
            u += (n_sp - 1) * ceil(wl.page_size, 64) + ceil(int(p["last_page_len"][i]), 64)
        units.append(u)
        qtiles.append(ceil(int(p["qo_indptr"][i + 1] - p["qo_indptr"][i]), 16))
    return units, qtiles


def _groups_of_plan(c, n):
    """Per stream (n_group, n_t32) from the plan image's stream records
    (20 ints each after an 8-int header; n_group at 10, n_t32 at 16)."""
    img = c.get_plan_image()
    recs = [img[8 + 20 * i: 8 + 20 * (i + 1)] for i in range(n)]
    return [int(r[10]) for r in recs], [int(r[16]) for r in recs], int(img[5])


@pytest.mark.parametrize("name", ["base", "r518", "frag"])
def test_split_counts_fill_one_round(name):
    """The planner's split counts keep every attention work-group of a run
    resident at once (at most the target count, which defaults to one per
    CU), and the stream with the longest splits (units per split times its
    busiest wave's tile-steps per unit), which sets the launch's length,
    could not take one more split that shortens them and still fit."""
    wl, c = _plan_at_measured_step(name)
    p = c.get_plan()
    shape = c.get_plan_shape()
    target = c.get_option(kvc.KVC_OPT_TARGET_WORKGROUPS)
    assert target == 256   # the CU count a metadata-only context assumes
    ceil = lambda a, b: -(-a // b)
    units, _ = _units_and_qtiles(wl, p)
    n_group, n_t32, shared = _groups_of_plan(c, len(units))
    heads = [wl.num_heads * g for g in n_group]
    ns = [int(x) for x in p["n_splits"]]
    items = sum(g * n for g, n in zip(heads, ns))
    assert items == shape["work_items"] <= target

    def per_unit(i):
        if wl.head_dim > 64:
            return 2.25 if shared else 2.0
        kmax = ceil(n_t32[i], n_group[i])
        return 2.0 * (kmax > 0) + 2.0 * (kmax > 4) + 0.25 * shared

    lens = [ceil(u, n) * per_unit(i) for i, (u, n) in enumerate(zip(units, ns))]
    i = lens.index(max(lens))
    u, g, n = units[i], heads[i], ns[i]
    if n < min(kvc.MAX_SPLITS, u) and ceil(u, n + 1) < ceil(u, n):
        assert items + g > target, (name, i, ns)


def test_f32_plan_has_no_splits():
    """Float32 pools: one work item (one wave) per 16-query tile and head,
    no KV split, hence no merge order; the 262-query frame of the base
    workload makes 17 tiles x 16 heads = 272 items."""
    wl = syn.WORKLOADS["base"]
    cfg = cfg_of(wl)
    cfg.dtype = kvc.KVC_DTYPE_F32
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    for _ in range(80):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
    assert list(c.get_plan()["n_splits"]) == [1]
    assert c.get_plan_shape() == {"work_items": 272, "group_rows": 16}
    img = c.get_plan_image()
    assert img[3] == 0 and img[5] == 0 and img[7] == 0   # no split, no shared tile, no merge slots


def test_query_grouping_choice():
    """A group of the 32x32 kernel is 4 waves x 2 tiles of 32 rows, plus, in
    a launch of the shared variant, a 16-row tail that the waves share (a
    quarter tile-step more per wave and unit).  The 262-query frame (8 full
    tiles and 6 rows) takes the tail: one group per head, 16 splits over 256
    work-groups, where 9 tiles would need two groups and half the splits.
    The 1005-query frame of the 999-patch workload (31 tiles and 13 rows)
    rounds up to 32 tiles: 4 groups of 8, 4 splits, no tail."""
    _, c = _plan_at_measured_step("base")
    assert c.get_plan_shape() == {"work_items": 256, "group_rows": 272}
    assert list(c.get_plan()["n_splits"]) == [16]
    _, c = _plan_at_measured_step("r518")
    assert c.get_plan_shape() == {"work_items": 256, "group_rows": 256}
    assert list(c.get_plan()["n_splits"]) == [4]


def test_scale_phase_multi_frame_steps_match_oracle():
    """A stream whose first step appends its S scale frames together ([p2]
    §Frame Processing Loop), then streams one frame per step; a second stream
    joins later with a 3-frame step.  Plans and counters bit-exact."""
    wl = syn.WORKLOADS["base"]
    c = cfg_of(wl)
    c.num_streams = 2
    c.max_patch_pages = 2 * (wl.scale_frames + wl.sliding_window + 16)
    c.max_special_pages = 12
    c.max_frames_per_step = wl.scale_frames
    cache = kvc.PagedKVCache(c, metadata_only=True)
    ocfg = ocfg_of(wl)
    ocfg.num_streams, ocfg.max_patch_pages, ocfg.max_special_pages = 2, c.max_patch_pages, 12
    ref = ko.AllocatorReplay(ocfg)
    for step in range(120):
        sched = {0: wl.scale_frames if step == 0 else 1}
        if step >= 30:
            sched[1] = 3 if step == 30 else 1
        active = sorted(sched)
        for s in active:
            cache.append_frames(0, num_frames=sched[s], stream_id=s)
            for _ in range(sched[s]):
                ref.append_frame(s)
        for s in active:
            cache.evict_frames(s)
            ref.evict_frames(s)
        cache.plan()
        ours = cache.get_plan()
        compare_plans(ours, ref.plan(active, [sched[s] for s in active]), active)
        for s in active:
            st = cache.get_cache_stats(s)
            theirs = ref.get_cache_stats(s)
            assert {k: st[k] for k in theirs} == theirs


def test_multi_frame_append_arguments_and_all_or_none():
    c = tiny_cache(num_blocks=2, max_frames_per_step=4)
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(0, num_frames=5)              # above max_frames_per_step
    assert e.value.status == kvc.KVC_ERR_ARG
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(0, num_frames=0)
    assert e.value.status == kvc.KVC_ERR_ARG
    c.append_frames(0, num_frames=3)
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(1, num_frames=2)              # differs from block 0
    assert e.value.status == kvc.KVC_ERR_ARG
    c.append_frames(1, num_frames=3)
    c.plan()
    assert list(c.get_plan()["qo_indptr"]) == [0, 3 * syn.WORKLOADS["tiny"].tokens_per_frame]
    # 6 patch pages: 3 used, a 4-frame step cannot fit and must leave no trace
    before = c.get_cache_stats()
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(0, num_frames=4)
    assert e.value.status == kvc.KVC_ERR_POOL_EXHAUSTED
    assert c.get_cache_stats() == before
    c.append_frames(0, num_frames=3)                  # exactly fills the pool
    assert c.get_cache_stats()["free_pages"] == 0


def test_rope_entry_points_on_metadata_only_context():
    """kvc_append_frames_rope follows kvc_append_frames' allocation and call
    order (a metadata-only context takes no tables); kvc_run_rope refuses to
    run without device buffers; the rope launch has its own profile slot."""
    lib = kvc.load_library()
    c = tiny_cache(num_blocks=2)
    fake = ctypes.c_void_p(16)
    rc = lib.kvc_append_frames_rope(c._ctx, 0, 0, None, None, 1, fake, fake, None)
    assert rc == kvc.KVC_ERR_ARG                       # tables on a metadata-only context
    assert lib.kvc_append_frames_rope(c._ctx, 0, 0, None, None, 1, None, None, None) == kvc.KVC_OK
    assert lib.kvc_append_frames_rope(c._ctx, 0, 0, None, None, 1, None, None, None) == kvc.KVC_ERR_STATE
    assert lib.kvc_append_frames_rope(c._ctx, 0, 1, None, None, 2, None, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_append_frames_rope(c._ctx, 0, 1, None, None, 1, None, None, None) == kvc.KVC_OK
    with pytest.raises(kvc.KvcError) as e:
        c.append_frames(0, num_frames=1, rope=(None, None))
    assert e.value.status == kvc.KVC_ERR_ARG
    assert lib.kvc_evict(c._ctx, 0) == kvc.KVC_OK
    assert lib.kvc_plan(c._ctx, None) == kvc.KVC_OK
    assert lib.kvc_run_rope(c._ctx, 0, fake, fake, fake, ctypes.c_void_p(4096), None) == kvc.KVC_ERR_STATE
    assert c.get_cache_stats()["frame_count"] == 1
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.kvc_profile_read(c._ctx, kvc.KVC_KERNEL_ROPE, ctypes.byref(ms), ctypes.byref(n), 0) == kvc.KVC_OK
    assert n.value == 0
    assert lib.kvc_profile_read(c._ctx, kvc.KVC_KERNEL_ROPE + 1, None, None, 0) == kvc.KVC_ERR_ARG


def test_deferred_eviction_and_rollback_match_oracle():
    """Rollback with deferred eviction (the reading of [p2] §Scale Frames vs
    Sliding Window): tables and counters bit-exact against the oracle's
    replay of the same rules, through every step, with rollbacks at seeded
    steps (scale frames included)."""
    wl = syn.WORKLOADS["base"]
    c = cfg_of(wl)
    cache = kvc.PagedKVCache(c, metadata_only=True)
    cache.set_option(kvc.KVC_OPT_DEFER_EVICTION, 1)
    assert cache.get_option(kvc.KVC_OPT_DEFER_EVICTION) == 1
    ref = ko.AllocatorReplay(ocfg_of(wl))
    ref.defer_eviction = True
    rng = np.random.default_rng(3)
    rolled = 0
    for step in range(150):
        cache.append_frame(0)
        ref.append_frame(0)
        cache.evict_frames()
        ref.evict_frames(0)
        cache.plan()
        compare_plans(cache.get_plan(), ref.plan([0]), [0])
        if rng.random() < 0.3 or step in (3, 7, 8):
            cache.rollback_frame(0)
            ref.rollback_frame(0)
            rolled += 1
            with pytest.raises(kvc.KvcError) as e:
                cache.rollback_frame(0)                   # only once per append
            assert e.value.status == kvc.KVC_ERR_STATE
        ours = cache.get_cache_stats(0)
        theirs = ref.get_cache_stats(0)
        assert {k: ours[k] for k in theirs} == theirs
    assert rolled > 20 and ours["frame_count"] == 150 - rolled


def test_rollback_errors():
    c = tiny_cache(num_blocks=2)
    c.append_frame(0)
    c.append_frame(1)
    c.evict_frames()
    c.plan()
    with pytest.raises(kvc.KvcError) as e:
        c.rollback_frame(0)                               # deferred eviction off
    assert e.value.status == kvc.KVC_ERR_STATE
    c.set_option(kvc.KVC_OPT_DEFER_EVICTION, 1)
    c.append_frame(0)
    with pytest.raises(kvc.KvcError) as e:
        c.rollback_frame(0)                               # inside a step
    assert e.value.status == kvc.KVC_ERR_STATE
    c.append_frame(1)
    c.evict_frames()
    c.plan()
    before = c.get_cache_stats()
    c.rollback_frame(0)
    after = c.get_cache_stats()
    assert after["frame_count"] == before["frame_count"] - 1
    assert after["special_tokens"] == before["special_tokens"] - syn.WORKLOADS["tiny"].num_special_tokens
    with pytest.raises(kvc.KvcError) as e:
        c.set_option(kvc.KVC_OPT_DEFER_EVICTION, 2)
    assert e.value.status == kvc.KVC_ERR_ARG


def test_build_refuses_kernels_that_spill():
    """The attention loop counts its own direct-to-LDS loads with vmcnt waits,
    so a build whose kernels use scratch memory is refused."""
    from paged_kv_cache_kvc_amd import build as b
    ok = ("k.hip:1:1: remark: Function Name: attn [-R]\nk.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-R]\n")
    b.check_no_scratch(ok)
    with pytest.raises(RuntimeError, match="attn2: 216"):
        b.check_no_scratch(ok + ok.replace("attn", "attn2").replace("]: 0", "]: 216"))
    # SGPR spills: refused in the kernel whose unit entries come from asm
    # scalar loads, accepted elsewhere
    spill = "k.hip:1:1: remark: Function Name: {} [-R]\nk.hip:1:1: remark:     SGPRs Spill: 15 [-R]\n"
    b.check_no_scratch(spill.format("_ZN3kvc13attn32_kernelILi64E"))
    with pytest.raises(RuntimeError, match="SGPRs spilled"):
        b.check_no_scratch(spill.format("_ZN3kvc11attn_kernelILi128E"))


def test_fused_append_option_and_plan():
    """KVC_OPT_FUSED_APPEND: 0 or 1 only; a plan built with it keeps the
    page tables, split counts and query grouping of the plain plan (only the
    unit table gains the cuts of the own rows, and the copy table follows
    the merge order); a metadata-only context has nothing to run."""
    wl = syn.WORKLOADS["base"]
    plain = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    fused = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    with pytest.raises(kvc.KvcError):
        fused.set_option(kvc.KVC_OPT_FUSED_APPEND, 2)
    fused.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    assert fused.get_option(kvc.KVC_OPT_FUSED_APPEND) == 1
    for _ in range(200):
        for c in (plain, fused):
            c.append_frame(0)
            c.evict_frames()
            c.plan()
    a, b = plain.get_plan(), fused.get_plan()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert plain.get_plan_shape() == fused.get_plan_shape()
    ia, ib = plain.get_plan_image(), fused.get_plan_image()
    T = wl.tokens_per_frame
    assert len(ib) >= len(ia) + T    # one pool row per input row after the merge order
    with pytest.raises(kvc.KvcError):
        fused.raw_run_append(0, [0], [0], 0, 0, 0)
