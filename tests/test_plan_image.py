"""Host-side checks of the device plan image: the int32 buffer that kvc_plan
uploads and the attention and merge kernels read without checks of their own
(the layout of paged_kv_cache_kvc_amd/csrc/kvc_plan_layout.h, restated here).

Each plan is decoded independently of the planner and checked against the
public plan (page tables, last-page lengths, query rows) and the pool
geometry: every work unit lies inside one visible page of its own stream, in
table order, within that page's valid slots, and the units add up to the
visible length; the splits of every work item tile the units; the merge order
lists each (query tile, head) of a split stream exactly once, on the XCD of
its middle split, with the tile's split count and output rows."""
import dataclasses
import math

import numpy as np
import pytest

import kvc_synth as syn
import paged_kv_cache_kvc_amd as kvc
from tests.stream_harness import edge_workloads
from tests.test_host_abi import cfg_of, free_orders

HEADER, REC, UNIT, MERGE, KV_TILE, XCD = 8, 20, 4, 4, 64, 8
Q_TILE32, TAIL_ROWS, WAVES32, Q_TILE16 = 32, 16, 4, 16
REC_FIELDS = ("q_row0", "n_q", "page0", "n_patch", "n_pages", "last_len", "kv_len", "unit0", "n_units",
              "n_split", "n_group", "item0", "n_items", "upp", "ups", "q_tile0", "n_t32", "tail",
              "reserved0", "reserved1")


def expected_grouping(wl, n_q, shared, k32):
    """(n_group, n_t32, tail) of a stream with n_q query rows.  With the
    32x32 kernel (D = 32 or 64) a group is 4 waves x 2 tiles of 32 rows; with
    the shared variant, rows past the last full tile form a 16-row tail of
    the last group when there are at most 16 of them.  With the 16x16 kernel
    (D = 128, or D = 64 when the plan takes it) a group is 8 tiles of 16
    rows, or 9 with the shared variant."""
    if k32:
        rem = n_q % Q_TILE32
        tail = 1 if shared and 1 <= rem <= TAIL_ROWS else 0
        nt = n_q // Q_TILE32 if tail else -(-n_q // Q_TILE32)
        return max(1, -(-nt // (2 * WAVES32))), nt, tail
    return -(-(-(-n_q // Q_TILE16)) // (9 if shared else 8)), 0, 0


def merge_group(r, t, k32):
    """The query group that computes (the first rows of) 32-row tile t."""
    if k32:
        if t >= r["n_t32"]:
            return r["n_group"] - 1
        return next(g for g in range(r["n_group"]) if t < (g + 1) * r["n_t32"] // r["n_group"])
    nqt = -(-r["n_q"] // Q_TILE16)
    return next(g for g in range(r["n_group"]) if 2 * t < (g + 1) * nqt // r["n_group"])


def check_image(wl, c, fused=False):
    img = c.get_plan_image().astype(np.int64)
    plan = c.get_plan()
    shape = c.get_plan_shape()
    H, pg = wl.num_heads, wl.page_size
    P = wl.tokens_per_frame - wl.num_special_tokens
    n_streams, n_items, n_rows, any_split, n_tiles, shared, merge_at, merge_slots = (int(x) for x in img[:HEADER])
    n = len(plan["planned"])
    assert n_streams == n
    # bit 0: the shared variant; bit 1: the 16x16 kernel at head_dim 64
    tiles16 = bool(shared & 2)
    shared &= 1
    assert img[5] in (0, 1, 2)
    assert not tiles16 or wl.head_dim == 64
    k32 = wl.head_dim <= 64 and not tiles16
    if k32:
        assert shape["group_rows"] == 2 * WAVES32 * Q_TILE32 + (TAIL_ROWS if shared else 0)
    else:
        assert shape["group_rows"] == (9 if shared else 8) * Q_TILE16
    assert n_items == shape["work_items"]
    assert n_rows == plan["qo_indptr"][-1]
    recs = [dict(zip(REC_FIELDS, (int(x) for x in img[HEADER + REC * i: HEADER + REC * (i + 1)]))) for i in range(n)]
    tables_at = HEADER + REC * n
    assert np.array_equal(img[tables_at: tables_at + len(plan["kv_indices"])], plan["kv_indices"])
    item = tiles = 0
    split_streams = set()
    fused_units = []
    for i, r in enumerate(recs):
        assert r["q_row0"] == plan["qo_indptr"][i] and r["n_q"] == plan["qo_indptr"][i + 1] - plan["qo_indptr"][i]
        assert r["page0"] == plan["kv_indptr"][i]
        assert r["n_pages"] == plan["kv_indptr"][i + 1] - plan["kv_indptr"][i]
        assert r["n_patch"] == plan["n_patch_pages"][i] and r["last_len"] == plan["last_page_len"][i]
        assert r["n_split"] == plan["n_splits"][i]
        assert r["reserved0"] == r["reserved1"] == 0
        # units: in table order, page by page, 64-slot chunks of each page's valid slots
        pages = plan["kv_indices"][r["page0"]: r["page0"] + r["n_pages"]]
        expect = []
        for pi, page in enumerate(pages):
            length = r["last_len"] if pi == r["n_pages"] - 1 else (P if pi < r["n_patch"] else pg)
            expect += [(int(page), s0, min(KV_TILE, length - s0)) for s0 in range(0, length, KV_TILE)]
        assert (r["n_units"] >= len(expect) if fused else r["n_units"] == len(expect)) and len(expect) >= 1
        assert r["unit0"] % 4 == 0
        got, srcs = [], []
        for u in range(r["n_units"]):
            slot, valid, z0, z1 = (int(x) for x in img[r["unit0"] + UNIT * u: r["unit0"] + UNIT * (u + 1)])
            page, s = divmod(slot & 0xFFFFFFFF, 2 * pg)   # pool rows [page][K, V][page_size]
            assert s < pg and z1 == 0 and (z0 >= 0 if fused else z0 == 0)
            got.append((page, s, valid))
            srcs.append(z0)
        if fused:
            # the 64-slot chunks, each cut into runs: the units tile every
            # chunk in order and none leaves its chunk
            joined = []
            for (page, s, valid) in got:
                assert valid >= 1 and s // KV_TILE == (s + valid - 1) // KV_TILE
                if joined and joined[-1][0] == page and joined[-1][1] + joined[-1][2] == s and s % KV_TILE:
                    joined[-1] = (page, joined[-1][1], joined[-1][2] + valid)
                else:
                    joined.append((page, s, valid))
            assert joined == expect
            fused_units.append((i, got, srcs))
        else:
            assert got == expect
        assert sum(v for _, _, v in got) == r["kv_len"]
        # work items: heads x splits x query groups, every split non-empty
        assert (r["n_group"], r["n_t32"], r["tail"]) == expected_grouping(wl, r["n_q"], shared, k32)
        if k32:
            assert all((g + 1) * r["n_t32"] // r["n_group"] - g * r["n_t32"] // r["n_group"] <= 2 * WAVES32
                       for g in range(r["n_group"]))
            assert 32 * r["n_t32"] + (TAIL_ROWS if r["tail"] else 0) >= r["n_q"] > 32 * r["n_t32"] - 32
        assert 1 <= r["n_split"] <= r["n_units"]
        assert r["n_split"] <= kvc.MAX_SPLITS or -(-r["n_units"] // kvc.MAX_SPLITS) > 512
        if k32:
            assert -(-r["n_units"] // r["n_split"]) <= 512   # a split's entries fit the kernel's LDS table
        bounds = [s * r["n_units"] // r["n_split"] for s in range(r["n_split"] + 1)]
        assert all(b1 > b0 for b0, b1 in zip(bounds, bounds[1:])) and bounds[-1] == r["n_units"]
        assert r["item0"] == item and r["n_items"] == H * r["n_split"] * r["n_group"]
        assert r["q_tile0"] == tiles
        item += r["n_items"]
        tiles += -(-r["n_q"] // Q_TILE32)
        if r["n_split"] > 1:
            split_streams.add(i)
    assert item == n_items and tiles == n_tiles and any_split == (1 if split_streams else 0)
    # merge order: one entry per (32-row tile, head) of a split stream
    merge_end = merge_at + MERGE * XCD * merge_slots
    if fused:
        check_copy_table(wl, c, img, recs, fused_units, -(-merge_end // 4) * 4, n_rows)
    else:
        assert len(img) == merge_end
    assert merge_at % 4 == 0
    ipx = -(-n_items // XCD)
    seen = {}
    for x in range(XCD):
        for k in range(merge_slots):
            e = [int(v) for v in img[merge_at + MERGE * (x * merge_slots + k): merge_at + MERGE * (x * merge_slots + k + 1)]]
            if e[0] < 0:
                continue
            assert e[0] not in seen
            seen[e[0]] = (x, e[1:])
    want = {}
    for i in split_streams:
        r = recs[i]
        for t in range(-(-r["n_q"] // Q_TILE32)):
            grp = merge_group(r, t, k32)
            for h in range(H):
                mid = r["item0"] + (h * r["n_split"] + r["n_split"] // 2) * r["n_group"] + grp
                want[(r["q_tile0"] + t) * H + h] = (min(mid // max(1, ipx), XCD - 1),
                                                    [r["n_split"], r["q_row0"] + Q_TILE32 * t,
                                                     min(Q_TILE32, r["n_q"] - Q_TILE32 * t)])
    assert seen == want


def check_copy_table(wl, c, img, recs, fused_units, at, n_rows):
    """Fused plans: after the merge order, the pool K row of every input row
    (the step's own frames, in query order).  Restated from the placement
    rules: frame f's patch row t (t outside the special rows) goes to slot
    t or t - n_s of the frame's patch page, which is the f-th of the last F
    patch pages of the table; its k-th special row to special position
    total - F n_s + f n_s + k of the stream's special pages.  A unit read
    from the input covers consecutive input rows whose pool rows are the
    unit's own; every other unit holds none of those pool rows."""
    assert len(img) == at + n_rows
    copy = img[at:].astype(np.int64) & 0xFFFFFFFF
    plan = c.get_plan()
    pg, T, ns, off = wl.page_size, wl.tokens_per_frame, wl.num_special_tokens, wl.row_offset
    for i, r in enumerate(recs):
        F = r["n_q"] // T
        pages = plan["kv_indices"][r["page0"]: r["page0"] + r["n_pages"]]
        sp_pages = pages[r["n_patch"]:]
        total_sp = sum(pg for _ in sp_pages[:-1]) + (r["last_len"] if len(sp_pages) else 0)
        own = copy[r["q_row0"]: r["q_row0"] + r["n_q"]]
        for f in range(F):
            patch_page = int(pages[r["n_patch"] - F + f])
            for t in range(T):
                if off <= t < off + ns:
                    pos = total_sp - F * ns + f * ns + (t - off)
                    want = int(sp_pages[pos // pg]) * 2 * pg + pos % pg
                else:
                    want = patch_page * 2 * pg + (t if t < off else t - ns)
                assert own[f * T + t] == want, (i, f, t)
        own_rows = {int(x): k for k, x in enumerate(own)}
        assert len(own_rows) == r["n_q"]
        for (si, got, srcs) in fused_units:
            if si != i:
                continue
            for (page, s, valid), z in zip(got, srcs):
                slot = page * 2 * pg + s
                if z:
                    assert z - 1 + valid <= r["n_q"]
                    assert all(own[z - 1 + k] == slot + k for k in range(valid))
                else:
                    assert all(slot + k not in own_rows for k in range(valid))


def stream_and_check(wl, steps_to_check, nframes=None):
    fp, fs = free_orders(wl)
    c = kvc.PagedKVCache(cfg_of(wl), metadata_only=True, free_patch_order=fp, free_special_order=fs) \
        if fp is not None else kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    F = max(wl.frames)
    starts = [F - f for f in wl.frames]
    for t in range(F):
        act = [s for s in range(len(wl.frames)) if t >= starts[s]]
        for s in act:
            c.append_frame(0, stream_id=s)
        for s in act:
            c.evict_frames(stream_id=s)
        c.plan()
        if t in steps_to_check or t == F - 1:
            check_image(wl, c)
    return c


@pytest.mark.parametrize("name", ["tiny", "base", "r518", "frag"])
def test_plan_image_workloads(name):
    wl = syn.WORKLOADS[name]
    F = max(wl.frames)
    stream_and_check(wl, set(range(F)) if name == "tiny" else {0, 1, wl.scale_frames, F // 2})


def test_plan_image_long_stream_tail():
    """10 000 frames: 235 special pages, the split bounds over 1228 units."""
    stream_and_check(syn.WORKLOADS["long"], {9998})


@pytest.mark.parametrize("name", sorted(edge_workloads()))
def test_plan_image_degenerate_shapes(name):
    wl = edge_workloads()[name]
    cfg = kvc.make_config(wl.num_blocks, wl.num_heads, wl.head_dim, wl.tokens_per_frame, wl.num_special_tokens,
                          page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                          num_streams=wl.num_streams, max_patch_pages=wl.max_patch_pages,
                          max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset,
                          max_frames_per_step=64)
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    done, first = 0, True
    while done < max(wl.frames):
        nf = min(64 if (first and name == "steps_of_64") else 1, max(wl.frames) - done)
        if nf > 1:
            c.append_frames(0, num_frames=nf)
        else:
            c.append_frame(0)
        c.evict_frames()
        c.plan()
        check_image(wl, c)
        done += nf
        first = False


def test_plan_image_check_catches_corruption():
    """The decoder above rejects a corrupted image: a unit moved by one slot,
    a valid count off by one, a work-item range shifted, a merge entry's
    rows or split count changed, a tile missing from the merge order."""
    wl = syn.WORKLOADS["tiny"]
    c = stream_and_check(wl, set())
    good = c.get_plan_image()
    plan = c.get_plan()
    n = len(plan["planned"])
    rec0 = HEADER
    unit0 = int(good[rec0 + REC_FIELDS.index("unit0")])
    merge_at, merge_slots = int(good[6]), int(good[7])
    first_merge = next(merge_at + MERGE * k for k in range(XCD * merge_slots) if good[merge_at + MERGE * k] >= 0)

    def corrupt(i, delta):
        bad = good.copy()
        bad[i] += delta
        return bad

    cases = [corrupt(unit0, 1), corrupt(unit0 + 2, -1), corrupt(rec0 + REC_FIELDS.index("item0"), 1),
             corrupt(first_merge + 1, 1), corrupt(first_merge + 2, 16)]
    missing = good.copy()
    missing[first_merge] = -1
    cases.append(missing)
    assert n == 1 and plan["n_splits"][0] > 1
    for bad in cases:
        c.get_plan_image = lambda bad=bad: bad
        with pytest.raises(AssertionError):
            check_image(wl, c)
    c.get_plan_image = lambda: good
    check_image(wl, c)


@pytest.mark.parametrize("tile", [16, 32])
@pytest.mark.parametrize("name", ["base", "tiny"])
def test_plan_image_forced_query_tile(name, tile):
    """KVC_OPT_QUERY_TILE fixes the head_dim 64 kernel: the image carries the
    16x16 bit exactly when 16 is asked for, over a scale step and steady
    steps."""
    wl = syn.WORKLOADS[name]
    c = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    c.set_option(kvc.KVC_OPT_QUERY_TILE, tile)
    assert c.get_option(kvc.KVC_OPT_QUERY_TILE) == tile
    for t in range(wl.scale_frames + 3):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
        check_image(wl, c)
        img = c.get_plan_image()
        assert bool(img[5] & 2) == (tile == 16 and wl.head_dim == 64)
        assert c.get_plan_shape()["group_rows"] == (128 if tile == 16 and wl.head_dim == 64 else 256 + 16 * (img[5] & 1))
    with pytest.raises(kvc.KvcError):
        c.set_option(kvc.KVC_OPT_QUERY_TILE, 64)


@pytest.mark.parametrize("heads,hist,nf,rows", [(16, 0, 8, 256), (32, 0, 8, 128), (16, 64, 1, 272),
                                                (8, 8, 1, 128), (2, 120, 1, 256)])
def test_planner_kernel_choice_head_dim_64(heads, hist, nf, rows):
    """The planner's choice between the two head_dim 64 kernels on a 256-CU
    target, at shapes where the faster one was measured: the 32x32 kernel for
    the one-frame steady state and the 16-head scale step; the 16x16 kernel
    for the 32-head scale step (the 32x32 kernel's 288 groups need a second
    round on 32 CUs) and for the short first steps over 8 heads.  The image
    is decoded and checked at every shape."""
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=heads)
    cfg = kvc.make_config(1, heads, 64, wl.tokens_per_frame, wl.num_special_tokens, page_size=wl.page_size,
                          scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                          max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages,
                          special_row_offset=wl.row_offset, max_frames_per_step=8)
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    c.set_option(kvc.KVC_OPT_TARGET_WORKGROUPS, 256)
    if hist:
        c.append_frames(0, num_frames=wl.scale_frames)
        c.evict_frames()
        c.plan()
        for _ in range(hist - wl.scale_frames):
            c.append_frame(0)
            c.evict_frames()
            c.plan()
    if nf > 1:
        c.append_frames(0, num_frames=nf)
    else:
        c.append_frame(0)
    c.evict_frames()
    c.plan()
    assert c.get_plan_shape()["group_rows"] == rows
    check_image(wl, c)


def _mid_specials():
    """Specials in the middle of the frame (rows 17..21 of 45): the patch
    rows of a frame are not consecutive in the input there."""
    return syn.Workload("mid_specials", 1, 2, 32, 40, 5, 64, 2, 6, (30,), 31,
                        max_patch_pages=2 + 6 + 1, max_special_pages=8, special_row_offset=17)


@pytest.mark.parametrize("name", ["tiny", "base", "r518", "mid_specials", "max_specials", "no_specials",
                                  "steps_of_64"])
def test_plan_image_fused_append(name):
    """Plans built for the fused append (KVC_OPT_FUSED_APPEND): the own
    frames' units and the copy table, on a scale step and single-frame
    steps."""
    wl = {"mid_specials": _mid_specials(), **edge_workloads()}.get(name) or syn.WORKLOADS[name]
    first = min(wl.scale_frames, 8) if name != "steps_of_64" else 64
    cfg = kvc.make_config(wl.num_blocks, wl.num_heads, wl.head_dim, wl.tokens_per_frame, wl.num_special_tokens,
                          page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                          num_streams=wl.num_streams, max_patch_pages=wl.max_patch_pages,
                          max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset,
                          max_frames_per_step=max(first, 1))
    c = kvc.PagedKVCache(cfg, metadata_only=True)
    c.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    F = min(max(wl.frames), 80)
    done = 0
    while done < F:
        nf = first if done == 0 and first > 1 else 1
        nf = min(nf, F - done)
        if nf > 1:
            c.append_frames(0, num_frames=nf)
        else:
            c.append_frame(0)
        c.evict_frames()
        c.plan()
        if done < 3 or done % 7 == 0 or done + nf == F:
            check_image(wl, c, fused=True)
        done += nf


def test_plan_image_fused_check_catches_corruption():
    """The fused decoder rejects a copy table entry moved by one row and an
    input row of a unit moved by one."""
    wl = syn.WORKLOADS["tiny"]
    c = kvc.PagedKVCache(cfg_of(wl), metadata_only=True)
    c.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    for _ in range(3):
        c.append_frame(0)
        c.evict_frames()
        c.plan()
    good = c.get_plan_image()
    check_image(wl, c, fused=True)
    n = len(c.get_plan()["planned"])
    rec0 = HEADER
    unit0, nu = int(good[rec0 + REC_FIELDS.index("unit0")]), int(good[rec0 + REC_FIELDS.index("n_units")])
    own = next(u for u in range(nu) if good[unit0 + UNIT * u + 2] > 0)
    bad1 = good.copy()
    bad1[-1] += 1
    bad2 = good.copy()
    bad2[unit0 + UNIT * own + 2] += 1
    assert n == 1
    for bad in (bad1, bad2):
        c.get_plan_image = lambda bad=bad: bad
        with pytest.raises(AssertionError):
            check_image(wl, c, fused=True)
