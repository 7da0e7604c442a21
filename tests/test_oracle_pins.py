"""Pins of the CPU oracle to facts outside itself (runs on CPU, no GPU).

Each pin is written as a function that raises AssertionError when the oracle
disagrees with: the worked example printed by [p3] 'How FlashInfer's Paged KV
Cache Attention Outperforms SDPA Fallback in Streaming Inference'
(§Inspecting Cache Statistics), closed forms of the append-only special
stream, the definition of the visible set, PyTorch's
scaled_dot_product_attention (an independent library routine), brute force
on tiny inputs, and softmax invariants.  The last tests plant plausible
mistakes in the oracle and check that some pin catches each one.
"""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

import kvc_synth as syn
from oracle import kvc_oracle as ko

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    wl = syn.WORKLOADS["tiny"]
    d = dict(num_heads=wl.num_heads, head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame,
             num_special_tokens=wl.num_special_tokens, page_size=wl.page_size,
             scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
             max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages)
    d.update(kw)
    return ko.OracleConfig(**d)


def rand_bits(rng, shape, scale=1.0):
    return syn.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def frame_source(cfg, seed, scale_q=1.0):
    cache = {}

    def kv(s, f, b):
        key = (s, f, b)
        if key not in cache:
            args = (cfg.tokens_per_frame, cfg.num_heads, cfg.head_dim, cfg.num_special_tokens, cfg.row_offset)
            cache[key] = (syn.frame_tensor(seed, s, f, b, "k", *args),
                          syn.frame_tensor(seed, s, f, b, "v", *args))
        return cache[key]

    def q(s, f, b):
        return syn.frame_tensor(seed, s, f, b, "q", cfg.tokens_per_frame, cfg.num_heads, cfg.head_dim,
                                cfg.num_special_tokens, cfg.row_offset, scale=scale_q)
    return kv, q


# --------------------------------------------------------------------------
# pins (each raises AssertionError on disagreement)
# --------------------------------------------------------------------------

def pin_worked_example(oracle=ko):
    with open(os.path.join(GOLDEN, "cache_stats_example.json")) as fh:
        g = json.load(fh)
    c = g["config"]
    cfg = oracle.OracleConfig(num_heads=1, head_dim=8, tokens_per_frame=c["tokens_per_frame"],
                              num_special_tokens=c["num_special_tokens"], page_size=c["page_size"],
                              scale_frames=c["scale_frames"], sliding_window=c["sliding_window"],
                              max_patch_pages=c["max_patch_pages"],
                              max_special_pages=-(-c["max_total_frames"] * c["num_special_tokens"] // c["page_size"]))
    a = oracle.AllocatorReplay(cfg)
    for _ in range(g["frames"]):
        a.append_frame(0)
        a.evict_frames(0)
    assert a.get_cache_stats(0) == g["expected"], (a.get_cache_stats(0), g["expected"])


def pin_special_closed_forms(oracle=ko):
    for n_s, pg, frames in [(6, 256, [1, 42, 200, 10000]), (6, 16, list(range(1, 13))),
                            (6, 1024, [500]), (6, 256, [50, 400, 1500, 4000]), (5, 7, list(range(1, 30)))]:
        F_max = max(frames)
        P = min(pg, 16)
        cfg = oracle.OracleConfig(num_heads=1, head_dim=8, tokens_per_frame=P + n_s,
                                  num_special_tokens=n_s, page_size=pg,
                                  scale_frames=1, sliding_window=2, max_patch_pages=4,
                                  max_special_pages=-(-F_max * n_s // pg))
        pg_eff = pg
        a = oracle.AllocatorReplay(cfg)
        for F in range(1, F_max + 1):
            a.append_frame(0)
            a.evict_frames(0)
            if F in frames:
                st = a.get_cache_stats(0)
                assert st["special_tokens"] == n_s * F
                plan = a.plan([0])
                assert plan["n_special_pages"][0] == -(-n_s * F // pg_eff)
                assert plan["last_page_len"][0] == ((n_s * F - 1) % pg_eff) + 1
    # values quoted for the benchmark workloads
    expect = {200: (5, 176), 10000: (235, 96), 50: (2, 44), 400: (10, 96), 1500: (36, 40), 4000: (94, 192)}
    for F, (pages, last) in expect.items():
        assert -(-6 * F // 256) == pages and ((6 * F - 1) % 256) + 1 == last


def pin_visible_set(oracle=ko, S=8, W=64, frames=300):
    cfg = oracle.OracleConfig(num_heads=1, head_dim=8, tokens_per_frame=262, num_special_tokens=6,
                              page_size=256, scale_frames=S, sliding_window=W, max_patch_pages=S + W + 1,
                              max_special_pages=-(-frames * 6 // 256))
    a = oracle.AllocatorReplay(cfg)
    for t in range(frames):
        a.append_frame(0)
        a.evict_frames(0)
        plan = a.plan([0])
        n_patch = int(plan["n_patch_pages"][0])
        assert n_patch == min(t + 1, S + W)
        vis = [f for f in range(t + 1) if f < S or f > t - W]          # independent definition
        pages_by_frame = [a.streams[0].frames[f].patch_page for f in vis]
        assert list(plan["kv_indices"][:n_patch]) == pages_by_frame
        # order scale -> window -> specials
        assert list(plan["kv_indices"][n_patch:]) == a.streams[0].all_special_pages
    assert n_patch == 72 or (S, W) != (8, 64)


def pin_sdpa(oracle=ko, seed=0):
    """oracle attention == PyTorch scaled_dot_product_attention (fp64, CPU)."""
    rng = np.random.default_rng(seed)
    for T, L, H, D, sc in [(22, 152, 2, 32, 1.0), (7, 300, 3, 64, 3.0), (5, 1, 1, 16, 1.0), (262, 700, 2, 64, 1.0)]:
        q, k, v = rand_bits(rng, (T, H, D), sc), rand_bits(rng, (L, H, D)), rand_bits(rng, (L, H, D))
        ours = oracle.attention_fp64(q, k, v)
        tq = torch.from_numpy(syn.bf16_bits_to_f32(q).astype(np.float64)).permute(1, 0, 2)[None]
        tk = torch.from_numpy(syn.bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)[None]
        tv = torch.from_numpy(syn.bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def pin_scale_phase(oracle=ko, seed=5):
    """[p2] §Frame Processing Loop: the scale phase runs one full attention
    pass over several initialization frames.  A first step that appends F
    frames and attends their F*T queries through the page table must equal
    PyTorch SDPA over the concatenated tokens of those frames (every query
    sees every token, its own frame's and the other frames' alike)."""
    cfg = tiny_cfg(scale_frames=3)
    T, H, D = cfg.tokens_per_frame, cfg.num_heads, cfg.head_dim
    rng = np.random.default_rng(seed)
    F = 3
    qs = [rand_bits(rng, (T, H, D), 2.0) for _ in range(F)]
    ks = [rand_bits(rng, (T, H, D)) for _ in range(F)]
    vs = [rand_bits(rng, (T, H, D)) for _ in range(F)]
    a = oracle.AllocatorReplay(cfg)
    pool = oracle.SimulatedPool(cfg)
    for f in range(F):
        pool.write_frame(a.append_frame(0), ks[f], vs[f])
    a.evict_frames(0)
    plan = a.plan([0], frames=[F])
    assert list(plan["qo_indptr"]) == [0, F * T]
    k, v = oracle.gather_paged(cfg, pool, plan, 0)
    assert k.shape[0] == F * T
    ours = oracle.attention_fp64(np.concatenate(qs), k, v)
    to = lambda b: torch.from_numpy(syn.bf16_bits_to_f32(b).astype(np.float64)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(to(np.concatenate(qs)), to(np.concatenate(ks)),
                                                           to(np.concatenate(vs)))[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def pin_rollback(oracle=ko, seed=7):
    """Deferred eviction for frame rollback ([p2] §Scale Frames vs Sliding
    Window): after undoing the latest frame, the paged view of the stream is
    the dense history of the frames it kept, as if the undone frame had never
    been appended; later frames stream on from there."""
    cfg = tiny_cfg(max_patch_pages=8, max_special_pages=8)
    T, H, D = cfg.tokens_per_frame, cfg.num_heads, cfg.head_dim
    rng = np.random.default_rng(seed)
    a = oracle.AllocatorReplay(cfg)
    a.defer_eviction = True
    pool = oracle.SimulatedPool(cfg)
    kept = []
    for i in range(24):
        k, v = rand_bits(rng, (T, H, D)), rand_bits(rng, (T, H, D))
        pool.write_frame(a.append_frame(0), k, v)
        kept.append((k, v))
        a.evict_frames(0)
        if i % 3 == 2 and i < 20:
            a.rollback_frame(0)
            kept.pop()
        plan = a.plan([0])
        kp, vp = oracle.gather_paged(cfg, pool, plan, 0)
        kd, vd = oracle.gather_dense(cfg, len(kept) - 1, lambda f: kept[f])
        assert np.array_equal(kp, kd) and np.array_equal(vp, vd)
        st = a.get_cache_stats(0)
        assert st["frame_count"] == len(kept)
        assert st["special_tokens"] == cfg.num_special_tokens * len(kept)


def pin_f16_inputs(oracle=ko, seed=11):
    """IEEE-half K/V/Q ([p3] §Precision and Hardware Utilization: the paged
    kernels take fp16 as well as bf16): the oracle on f16 bit patterns equals
    PyTorch SDPA in float64 over torch's own decoding of the same halves, and
    differs from reading those bits as bf16."""
    rng = np.random.default_rng(seed)
    T, L, H, D = 9, 40, 2, 32
    q, k, v = (syn.f32_to_f16_bits(rng.standard_normal(sh).astype(np.float32) * np.float32(sc))
               for sh, sc in (((T, H, D), 1.5), ((L, H, D), 1.0), ((L, H, D), 1.0)))
    ours = oracle.attention_fp64(q, k, v, "f16")
    to = lambda b: torch.from_numpy(b.view(np.float16)).double().permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(to(q), to(k), to(v))[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def pin_f32_inputs(oracle=ko, seed=12):
    """float32 K/V/Q (a full-precision pool): the oracle on f32 bit patterns
    equals PyTorch SDPA in float64 over the same float32 values, and differs
    from reading the high halves of those bits as bf16."""
    rng = np.random.default_rng(seed)
    T, L, H, D = 7, 33, 2, 32
    q, k, v = (syn.f32_to_bits(rng.standard_normal(sh).astype(np.float32) * np.float32(sc), "f32")
               for sh, sc in (((T, H, D), 1.5), ((L, H, D), 1.0), ((L, H, D), 1.0)))
    assert q.dtype == np.uint32
    ours = oracle.attention_fp64(q, k, v, "f32")
    to = lambda b: torch.from_numpy(b.view(np.float32)).double().permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(to(q), to(k), to(v))[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def pin_round_to_f32(oracle=ko, seed=14):
    """round_to_elem for f32 is nearest-even: every result is one of the two
    float32 neighbours of the value (found with nextafter), the nearer one;
    exact midpoints go to the even pattern, and values a hair past a
    midpoint to the far side."""
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(3000) * np.exp2(rng.uniform(-40, 40, 3000))).astype(np.float32)
    b = np.nextafter(a, np.float32(np.inf))
    mid = 0.5 * (a.astype(np.float64) + b.astype(np.float64))       # exact in float64
    up = mid + np.abs(mid) * 2.0 ** -45
    x = mid + (b.astype(np.float64) - a.astype(np.float64)) * rng.uniform(-0.49, 0.49, 3000)
    got = oracle.round_to_elem(x, "f32").view(np.float32)
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    d_lo, d_hi = np.abs(x - lo), np.abs(x - hi)
    want = np.where(d_lo < d_hi, lo, hi)
    assert np.array_equal(got, want.astype(np.float32))
    tie = oracle.round_to_elem(mid, "f32")
    even = np.where(a.view(np.uint32) % 2 == 0, a, b).view(np.uint32)
    assert np.array_equal(tie, even)
    assert np.array_equal(oracle.round_to_elem(up, "f32").view(np.float32), np.where(up > mid, hi, lo))


def pin_bruteforce(oracle=ko, seed=1):
    """Scalar loops straight from the definition of softmax attention."""
    rng = np.random.default_rng(seed)
    T, L, H, D = 3, 5, 2, 4
    q, k, v = rand_bits(rng, (T, H, D), 2.0), rand_bits(rng, (L, H, D)), rand_bits(rng, (L, H, D))
    Q, K, V = (syn.bf16_bits_to_f32(x).astype(float).tolist() for x in (q, k, v))
    out = oracle.attention_fp64(q, k, v)
    for i in range(T):
        for h in range(H):
            logits = [sum(Q[i][h][d] * K[j][h][d] for d in range(D)) / math.sqrt(D) for j in range(L)]
            w = [math.exp(x) for x in logits]
            z = sum(w)
            for d in range(D):
                o = sum(w[j] * V[j][h][d] for j in range(L)) / z
                assert abs(o - out[i, h, d]) < 1e-12


def pin_lse_base2(oracle=ko, seed=3):
    """lse_base2_fp64 = log2 sum_j exp(q.k_j / sqrt(D)): a scalar loop from the
    definition on tiny inputs, PyTorch's logsumexp in float64 divided by ln 2
    as a second routine, and the split-KV identity it exists for: attention
    over chunks of the keys, merged with weights 2^(lse_c - lse), equals
    attention over all keys, and log2 of the sum of 2^lse_c equals lse."""
    import torch
    rng = np.random.default_rng(seed)
    T, L, H, D = 3, 7, 2, 4
    q, k = rand_bits(rng, (T, H, D), 2.0), rand_bits(rng, (L, H, D))
    Q, K = (syn.bf16_bits_to_f32(x).astype(float).tolist() for x in (q, k))
    lse = oracle.lse_base2_fp64(q, k)
    assert lse.shape == (T, H)
    for i in range(T):
        for h in range(H):
            z = sum(math.exp(sum(Q[i][h][d] * K[j][h][d] for d in range(D)) / math.sqrt(D)) for j in range(L))
            assert abs(math.log2(z) - lse[i, h]) < 1e-12
    T, L, H, D = 6, 50, 3, 32
    q, k, v = rand_bits(rng, (T, H, D), 1.5), rand_bits(rng, (L, H, D)), rand_bits(rng, (L, H, D))
    qd, kd = (torch.from_numpy(syn.bf16_bits_to_f32(x).astype(np.float64)) for x in (q, k))
    s = torch.einsum("thd,lhd->thl", qd, kd) / math.sqrt(D)
    ref = (torch.logsumexp(s, dim=2) / math.log(2.0)).numpy()
    np.testing.assert_allclose(oracle.lse_base2_fp64(q, k), ref, rtol=0, atol=1e-12)
    full = oracle.attention_fp64(q, k, v)
    lse = oracle.lse_base2_fp64(q, k)
    cuts = [0, 11, 12, 30, 50]
    parts = [(oracle.attention_fp64(q, k[a:b], v[a:b]), oracle.lse_base2_fp64(q, k[a:b]))
             for a, b in zip(cuts[:-1], cuts[1:])]
    merged = sum(o * np.exp2(l - lse)[:, :, None] for o, l in parts)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.log2(sum(np.exp2(l) for _, l in parts)), lse, rtol=0, atol=1e-12)


def pin_softmax_invariants(oracle=ko, seed=2):
    rng = np.random.default_rng(seed)
    T, L, H, D = 9, 40, 2, 32
    q, k = rand_bits(rng, (T, H, D)), rand_bits(rng, (L, H, D))
    c = syn.f32_to_bf16_bits(np.full((L, H, D), 0.7109375, np.float32))    # exactly representable
    o = oracle.attention_fp64(q, k, c)
    np.testing.assert_allclose(o, 0.7109375, rtol=0, atol=1e-14)
    # planted key k* = alpha * q_0 dominates query row 0
    v = rand_bits(rng, (L, H, D))
    qf = syn.bf16_bits_to_f32(q)
    k2 = k.copy()
    k2[17] = syn.f32_to_bf16_bits(qf[0] * 8.0)
    o = oracle.attention_fp64(q, k2, v)
    np.testing.assert_allclose(o[0], syn.bf16_bits_to_f32(v[17]), atol=1e-6)
    # joint permutation of keys and values
    perm = rng.permutation(L)
    o1 = oracle.attention_fp64(q, k, v)
    o2 = oracle.attention_fp64(q, k[perm], v[perm])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    # a query of zeros averages the values uniformly
    qz = np.zeros_like(q)
    np.testing.assert_allclose(oracle.attention_fp64(qz, k, v),
                               np.broadcast_to(syn.bf16_bits_to_f32(v).astype(np.float64).mean(0), (T, H, D)),
                               atol=1e-14)


def pin_paged_equals_dense(oracle=ko, cfg=None, frames=12, seed=0, orders=(None, None), check_every=1):
    """Paged attention over the simulated pool == dense attention over the
    history gathered from the definition of the visible set (bitwise)."""
    cfg = cfg or tiny_cfg()
    kv, q = frame_source(cfg, seed)
    o = oracle.OracleStream(cfg, blocks=(0,), free_patch_order=orders[0], free_special_order=orders[1])
    outs = []
    for t in range(frames):
        plan = o.step([0], kv)
        if t % check_every and t != frames - 1:
            continue
        qb = q(0, t, 0)
        paged = o.attend(plan, 0, qb)
        kd, vd = oracle.gather_dense(cfg, t, lambda f: kv(0, f, 0))
        dense = oracle.attention_fp64(qb, kd, vd)
        assert np.array_equal(paged, dense), f"step {t}"
        outs.append(paged)
    return outs


# --------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------

def test_worked_example_cache_stats():
    pin_worked_example()


def test_special_stream_closed_forms():
    pin_special_closed_forms()


def test_visible_set_and_order():
    pin_visible_set()
    pin_visible_set(S=1, W=4, frames=40)


def test_attention_matches_torch_sdpa():
    pin_sdpa()


def test_scale_phase_multi_frame_step_is_dense_sdpa():
    pin_scale_phase()


def test_rollback_leaves_the_kept_frames_history():
    pin_rollback()


def test_f16_inputs_match_torch_sdpa():
    pin_f16_inputs()


def test_f32_inputs_match_torch_sdpa():
    pin_f32_inputs()


def test_round_to_f32_is_nearest_even():
    pin_round_to_f32()


def test_attention_bruteforce():
    pin_bruteforce()


def test_lse_base2_definition_and_split_identity():
    pin_lse_base2()


def test_softmax_invariants():
    pin_softmax_invariants()


def test_paged_equals_dense_tiny():
    pin_paged_equals_dense()


def test_paged_equals_dense_base_shape():
    # base page geometry (256 patches + 6 specials, S=8, W=64) at reduced H, D
    cfg = ko.OracleConfig(num_heads=1, head_dim=16, tokens_per_frame=262, num_special_tokens=6, page_size=256,
                          scale_frames=8, sliding_window=64, max_patch_pages=88, max_special_pages=4)
    pin_paged_equals_dense(cfg=cfg, frames=150, check_every=37)


def test_padded_patch_pages_equal_dense():
    # page_size > P: 13 patches in 16-slot pages (pad slots never attended)
    cfg = ko.OracleConfig(num_heads=2, head_dim=16, tokens_per_frame=19, num_special_tokens=6, page_size=16,
                          scale_frames=2, sliding_window=3, max_patch_pages=6, max_special_pages=10)
    pin_paged_equals_dense(cfg=cfg, frames=20)


def test_specials_first_row_layout():
    cfg = tiny_cfg(special_row_offset=0)
    pin_paged_equals_dense(cfg=cfg, frames=12)


def test_page_permutation_invariance():
    cfg = tiny_cfg()
    base = pin_paged_equals_dense(cfg=cfg, frames=12)
    po = syn.free_list_order(7, cfg.max_patch_pages, 0, 0)
    so = syn.free_list_order(7, cfg.max_special_pages, cfg.max_patch_pages, 1)
    assert list(po) != list(range(cfg.max_patch_pages))
    perm = pin_paged_equals_dense(cfg=cfg, frames=12, orders=(po, so))
    for a, b in zip(base, perm):
        assert np.array_equal(a, b)


def test_single_frame_reduces_to_sdpa():
    cfg = tiny_cfg()
    kv, q = frame_source(cfg, 3)
    o = ko.OracleStream(cfg)
    plan = o.step([0], kv)
    qb = q(0, 0, 0)
    out = o.attend(plan, 0, qb)
    k, v = kv(0, 0, 0)
    sel = np.concatenate([syn.patch_rows(22, 6, 16), syn.special_rows(22, 6, 16)])
    tq, tk, tv = (torch.from_numpy(syn.bf16_bits_to_f32(x).astype(np.float64)).permute(1, 0, 2)[None]
                  for x in (qb, k[sel], v[sel]))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_tiny_boundary_cases():
    cfg = tiny_cfg()
    a = ko.AllocatorReplay(cfg)
    seen_full_tail = seen_straddle = seen_reuse = False
    last_freed = []
    for t in range(12):
        fs = a.append_frame(0)
        if last_freed:
            # one spare page beyond S+W: the page freed last step is the one reused now
            assert fs.patch_page == last_freed[0]
            seen_reuse = True
        pages = {p for p, _ in fs.special}
        if len(pages) == 2:
            seen_straddle = True
            if t == 2:      # tokens 12..17: slots 12..15 of one page, 0..1 of the next
                assert [s for _, s in fs.special] == [12, 13, 14, 15, 0, 1]
        last_freed = a.evict_frames(0)
        plan = a.plan([0])
        if plan["last_page_len"][0] == cfg.page_size:
            seen_full_tail = True
            assert t == 7
    assert seen_full_tail and seen_straddle and seen_reuse


def test_conservation_and_uniqueness_multi_stream():
    wl = syn.WORKLOADS["frag"]
    cfg = ko.OracleConfig(num_heads=1, head_dim=8, tokens_per_frame=wl.tokens_per_frame,
                          num_special_tokens=6, page_size=256, scale_frames=wl.scale_frames,
                          sliding_window=wl.sliding_window, max_patch_pages=wl.max_patch_pages,
                          max_special_pages=wl.max_special_pages, num_streams=4)
    a = ko.AllocatorReplay(cfg, syn.free_list_order(wl.seed, wl.max_patch_pages, 0, 0),
                           syn.free_list_order(wl.seed, wl.max_special_pages, wl.max_patch_pages, 1))
    total = max(wl.frames)
    for step in range(total):
        active = [s for s in range(4) if step >= syn.stream_join_step(wl, s)]
        for s in active:
            a.append_frame(s)
        for s in active:
            a.evict_frames(s)
        if step % 97 == 0 or step == total - 1:
            plan = a.plan(active)
            idx = plan["kv_indices"]
            assert len(set(idx.tolist())) == len(idx)
            held = sum(len(a.streams[s].scale_patch_pages) + len(a.streams[s].live_window_patch_pages)
                       for s in range(4))
            assert held + len(a.free_patch_pages) == cfg.max_patch_pages
            held_sp = sum(len(a.streams[s].all_special_pages) for s in range(4))
            assert held_sp + len(a.free_special_pages) == cfg.max_special_pages
    assert [a.streams[s].frame_count for s in range(4)] == list(wl.frames)
    # free special pool is exactly used up by the sizing rule
    assert len(a.free_special_pages) == 0


def test_streams_are_independent():
    # two streams sharing one pool and free lists attend exactly as alone
    cfg = tiny_cfg(num_streams=2, max_patch_pages=12, max_special_pages=10)
    kv, q = frame_source(cfg, 5)
    both = ko.OracleStream(cfg)
    solo_cfg = tiny_cfg()
    for t in range(12):
        plan = both.step([0, 1], kv)
        qb = np.concatenate([q(0, t, 0), q(1, t, 0)])
        out = both.attend(plan, 0, qb)
        for s in range(2):
            kd, vd = ko.gather_dense(solo_cfg, t, lambda f: kv(s, f, 0))
            ref = ko.attention_fp64(q(s, t, 0), kd, vd)
            assert np.array_equal(out[s * 22:(s + 1) * 22], ref)


def test_pool_exhaustion_leaves_state_unchanged():
    cfg = tiny_cfg(max_special_pages=3)      # 48 special slots: 8 frames of 6
    a = ko.AllocatorReplay(cfg)
    for _ in range(8):
        a.append_frame(0)
        a.evict_frames(0)
    before = (a.get_cache_stats(0), list(a.free_patch_pages), list(a.free_special_pages))
    with pytest.raises(ko.PoolExhausted):
        a.append_frame(0)
    assert (a.get_cache_stats(0), list(a.free_patch_pages), list(a.free_special_pages)) == before


def test_constant_footprint_long_stream():
    wl = syn.WORKLOADS["long"]
    cfg = ko.OracleConfig(num_heads=wl.num_heads, head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame,
                          num_special_tokens=6, page_size=256, scale_frames=8, sliding_window=64,
                          max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages)
    before = ko.pool_bytes(cfg, wl.num_blocks)
    a = ko.AllocatorReplay(cfg)
    for t in range(10000):
        a.append_frame(0)
        a.evict_frames(0)
        assert len(a.streams[0].live_window_patch_pages) <= 64
        assert len(a.free_patch_pages) >= 88 - 72 - 1
    plan = a.plan([0])
    assert plan["n_patch_pages"][0] == 72 and plan["n_special_pages"][0] == 235
    assert plan["last_page_len"][0] == 96
    assert ko.pool_bytes(cfg, wl.num_blocks) == before == 24 * (88 + 235) * 2 * 256 * 16 * 64 * 2


def test_reset_replays_identically():
    cfg = tiny_cfg()
    a = ko.AllocatorReplay(cfg)
    first = []
    for _ in range(9):
        a.append_frame(0)
        a.evict_frames(0)
        first.append({k: v.tolist() for k, v in a.plan([0]).items()})
    a.reset()
    for i in range(9):
        a.append_frame(0)
        a.evict_frames(0)
        assert {k: v.tolist() for k, v in a.plan([0]).items()} == first[i]


# --------------------------------------------------------------------------
# rotary embedding pins ([p2] "How LingBot-Map Uses FlashInfer KV Cache for
# Streaming 3D Reconstruction" §3D RoPE Position Encoding): rounding by brute
# force over every 16-bit pattern, rotations with known results, complex
# multiplication as a second routine, and the two properties that make a
# rotary embedding one (norm preservation, relative position)
# --------------------------------------------------------------------------

def _elem_table(dtype):
    """Every finite non-negative value of the element type, ascending, with
    its bit pattern."""
    bits = np.arange(0x8000, dtype=np.uint32)
    if dtype == "bf16":
        with np.errstate(invalid="ignore"):
            vals = (bits << 16).view(np.float32).astype(np.float64)
    else:
        vals = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    return vals[ok], bits[ok].astype(np.uint16)


def _nearest_elem(x, dtype):
    """IEEE round-to-nearest-even by search: the closest table value, the one
    with an even bit pattern when two are equally close."""
    vals, bits = _elem_table(dtype)
    ax = np.abs(np.asarray(x, dtype=np.float64)).ravel()
    hi = np.clip(np.searchsorted(vals, ax), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = ax - vals[lo], vals[hi] - ax
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(bits[lo] % 2 == 0, lo, hi)))
    out = bits[pick] | np.where(np.signbit(np.asarray(x, dtype=np.float64).ravel()), 0x8000, 0).astype(np.uint16)
    return out.reshape(np.shape(x))


def _rope_inputs(seed, T=6, H=3, D=16, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, D)) * 2.0
    bits = syn.f32_to_bits(x.astype(np.float32), "f32") if dtype == "f32" else _nearest_elem(x, dtype)
    theta = rng.uniform(-4 * math.pi, 4 * math.pi, (T, D // 2))
    return bits, theta


def pin_round_to_elem(oracle=ko, seed=13):
    """round_to_elem is IEEE nearest-even, found by brute force: random values
    over 60 binades, exact midpoints between neighbours (ties to the even
    pattern), and values a hair past a midpoint, where rounding first to
    float32 and then to bf16 would land on the tie and round the wrong way."""
    rng = np.random.default_rng(seed)
    for dtype, emax in (("bf16", 30), ("f16", 14)):
        vals, _ = _elem_table(dtype)
        x = rng.choice([-1.0, 1.0], 4000) * np.exp2(rng.uniform(-emax, emax, 4000))
        normal = vals[(vals >= 2.0 ** -emax) & (vals < 2.0 ** emax)]
        i = rng.integers(0, len(normal) - 1, 2000)
        mid = 0.5 * (normal[i] + normal[i + 1])                     # exact in float64
        hair = mid + np.ldexp(np.abs(mid), -40) * rng.choice([-1.0, 1.0], 2000)
        for xs in (x, mid, -mid, hair, -hair, normal[i], -normal[i]):
            got = oracle.round_to_elem(xs, dtype)
            assert got.dtype == np.uint16 and np.array_equal(got, _nearest_elem(xs, dtype)), dtype


def pin_rope_known_rotations(oracle=ko, seed=17):
    """R_0 = I leaves every bit unchanged; a quarter turn maps (a, b) to
    (-b, a) and a half turn to (-a, -b), exactly, for every element type;
    rope_fp64 is the rotation rounded once to the nearest element value (the
    16-bit types by brute force here, f32 through pin_round_to_f32)."""
    for dtype in ("bf16", "f16", "f32"):
        bits, theta = _rope_inputs(seed, dtype=dtype)
        x = syn.bits_to_f32(bits, dtype).astype(np.float64)
        one, zero = np.ones_like(theta), np.zeros_like(theta)
        assert np.array_equal(oracle.rope_fp64(bits, one, zero, dtype), bits)
        quarter = oracle.rope_rotate_fp64(bits, zero, one, dtype)
        assert np.array_equal(quarter[..., 0::2], -x[..., 1::2]) and np.array_equal(quarter[..., 1::2], x[..., 0::2])
        half = oracle.rope_rotate_fp64(bits, -one, zero, dtype)
        assert np.array_equal(half, -x)
        c, s = np.cos(theta), np.sin(theta)
        if dtype != "f32":
            assert np.array_equal(oracle.rope_fp64(bits, c, s, dtype),
                                  _nearest_elem(oracle.rope_rotate_fp64(bits, c, s, dtype), dtype))


def pin_rope_complex(oracle=ko, seed=19):
    """Each pair (x[2i], x[2i+1]) read as a complex number and multiplied by
    cos(theta) + i sin(theta), with NumPy's complex arithmetic."""
    bits, theta = _rope_inputs(seed, T=9, H=4, D=32)
    x = syn.bits_to_f32(bits, "bf16").astype(np.float64)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (np.cos(theta) + 1j * np.sin(theta))[:, None, :]
    got = oracle.rope_rotate_fp64(bits, np.cos(theta), np.sin(theta))
    assert np.allclose(got[..., 0::2], z.real, rtol=0, atol=1e-14)
    assert np.allclose(got[..., 1::2], z.imag, rtol=0, atol=1e-14)


def pin_rope_norm_and_relative_position(oracle=ko, seed=23, D=32, base=10000.0):
    """With angles theta[t, i] = p_t * w_i (one frequency per pair), the
    rotation keeps every pair's length, and the score of a rotated query
    against a rotated key depends only on the position difference:
    <R(p) q, R(p') k> = <q, R(p' - p) k>."""
    rng = np.random.default_rng(seed)
    T, H = 12, 3
    w = base ** (-np.arange(D // 2) * 2.0 / D)
    pq, pk = rng.integers(0, 5000, T), rng.integers(0, 5000, T)
    qb = _nearest_elem(rng.standard_normal((T, H, D)), "bf16")
    kb = _nearest_elem(rng.standard_normal((T, H, D)), "bf16")

    def rot(bits, pos):
        ang = pos[:, None] * w[None, :]
        return oracle.rope_rotate_fp64(bits, np.cos(ang), np.sin(ang))
    q = syn.bits_to_f32(qb, "bf16").astype(np.float64)
    rq = rot(qb, pq)
    n0 = q[..., 0::2] ** 2 + q[..., 1::2] ** 2
    assert np.allclose(rq[..., 0::2] ** 2 + rq[..., 1::2] ** 2, n0, rtol=1e-13, atol=0)
    lhs = np.einsum("thd,thd->th", rq, rot(kb, pk))
    rhs = np.einsum("thd,thd->th", q, rot(kb, pk - pq))
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)


def test_round_to_elem_is_nearest_even():
    pin_round_to_elem()


def test_rope_known_rotations():
    pin_rope_known_rotations()


def test_rope_is_complex_multiplication():
    pin_rope_complex()


def test_rope_norm_and_relative_position():
    pin_rope_norm_and_relative_position()


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# --------------------------------------------------------------------------

class _Mutant:
    """A copy of the oracle module's namespace with one function replaced."""

    def __init__(self, **overrides):
        self.__dict__.update({k: getattr(ko, k) for k in dir(ko) if not k.startswith("__")})
        self.__dict__.update(overrides)


def _no_scale(q_bits, k_bits, v_bits, dtype="bf16"):
    q = syn.bf16_bits_to_f32(q_bits).astype(np.float64)
    k = syn.bf16_bits_to_f32(k_bits).astype(np.float64)
    v = syn.bf16_bits_to_f32(v_bits).astype(np.float64)
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        s = q[:, h, :] @ k[:, h, :].T
        p = np.exp(s - s.max(1, keepdims=True))
        out[:, h, :] = (p / p.sum(1, keepdims=True)) @ v[:, h, :]
    return out


def _values_are_keys(q_bits, k_bits, v_bits, dtype="bf16"):
    return ko.attention_fp64(q_bits, k_bits, k_bits, dtype)


def _f16_read_as_bf16(q_bits, k_bits, v_bits, dtype="bf16"):
    return ko.attention_fp64(q_bits, k_bits, v_bits)   # ignores the element type


def _sum_over_queries(q_bits, k_bits, v_bits, dtype="bf16"):
    q = syn.bf16_bits_to_f32(q_bits).astype(np.float64)
    k = syn.bf16_bits_to_f32(k_bits).astype(np.float64)
    v = syn.bf16_bits_to_f32(v_bits).astype(np.float64)
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        s = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(q.shape[2])
        p = np.exp(s - s.max(0, keepdims=True))
        p = p / p.sum(0, keepdims=True)          # normalised over the wrong axis
        out[:, h, :] = p @ v[:, h, :]
    return out


class _OffByOneWindow(ko.AllocatorReplay):
    def evict_frames(self, stream):
        st = self.streams[stream]
        while len(st.live_window_patch_pages) > self.cfg.sliding_window - 1:
            self.free_patch_pages.append(st.live_window_patch_pages.popleft())


class _SpecialsFirst(ko.AllocatorReplay):
    def build_visible_page_table(self, stream):
        st = self.streams[stream]
        return list(st.all_special_pages) + list(st.scale_patch_pages) + list(st.live_window_patch_pages)


class _LastPageZeroWhenFull(ko.AllocatorReplay):
    def compute_last_page_len(self, stream):
        return super().compute_last_page_len(stream) % self.cfg.page_size


class _ScaleEvicted(ko.AllocatorReplay):
    def append_frame(self, stream):
        fs = super().append_frame(stream)
        st = self.streams[stream]
        if len(st.scale_patch_pages) == self.cfg.scale_frames and st.frame_count == self.cfg.scale_frames:
            # wrongly treat scale frames as ordinary window frames
            st.live_window_patch_pages.extendleft(reversed(st.scale_patch_pages))
            st.scale_patch_pages.clear()
        return fs


class _OneFramePerStep(ko.AllocatorReplay):
    def plan(self, streams, frames=None):
        return super().plan(streams)      # ignores the frames of a scale-phase step


class _RollbackKeepsHeldBack(ko.AllocatorReplay):
    def rollback_frame(self, stream):
        st = self.streams[stream]
        held, st.held_back = st.held_back, []
        fs = super().rollback_frame(stream)   # window not refilled
        self.free_patch_pages.extend(held)
        return fs


class _LifoSpecialReuse(ko.AllocatorReplay):
    def append_frame(self, stream):
        fs = super().append_frame(stream)
        self.streams[stream].special_tokens += 0 if fs.patch_page % 2 else 1   # drifts the special count
        return fs


def _lse_natural_log(q_bits, k_bits, dtype="bf16"):
    return ko.lse_base2_fp64(q_bits, k_bits, dtype) * math.log(2.0)    # forgets the base change


def _lse_max_only(q_bits, k_bits, dtype="bf16"):
    q = syn.bf16_bits_to_f32(q_bits).astype(np.float64)
    k = syn.bf16_bits_to_f32(k_bits).astype(np.float64)
    return np.stack([((q[:, h] @ k[:, h].T) / math.sqrt(q.shape[2])).max(1) for h in range(q.shape[1])],
                    1) / math.log(2.0)


def _lse_unscaled(q_bits, k_bits, dtype="bf16"):
    q = syn.bf16_bits_to_f32(q_bits).astype(np.float64)
    k = syn.bf16_bits_to_f32(k_bits).astype(np.float64)
    out = np.empty(q.shape[:2])
    for h in range(q.shape[1]):
        s = q[:, h] @ k[:, h].T                   # no 1/sqrt(D)
        m = s.max(1)
        out[:, h] = (m + np.log(np.exp(s - m[:, None]).sum(1))) / math.log(2.0)
    return out


def _rope_parts(x_bits, cos, sin, dtype):
    x = syn.bits_to_f32(x_bits, dtype).astype(np.float64)
    T, H, D = x.shape
    return x, np.asarray(cos, np.float64).reshape(T, 1, D // 2), np.asarray(sin, np.float64).reshape(T, 1, D // 2)


def _rope_sign_slip(x_bits, cos, sin, dtype="bf16"):
    x, c, s = _rope_parts(x_bits, cos, sin, dtype)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s      # + where - belongs
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _rope_dropped_term(x_bits, cos, sin, dtype="bf16"):
    x, c, s = _rope_parts(x_bits, cos, sin, dtype)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 1::2] * c                         # a sin dropped
    return out


def _rope_rotate_half(x_bits, cos, sin, dtype="bf16"):
    x, c, s = _rope_parts(x_bits, cos, sin, dtype)
    h = x.shape[2] // 2
    a, b = x[..., :h], x[..., h:]                             # pairs (i, i + D/2)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=2)


def _rope_inverse(x_bits, cos, sin, dtype="bf16"):
    x, c, s = _rope_parts(x_bits, cos, sin, dtype)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s      # turns by -theta
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _f32_read_as_bf16(q_bits, k_bits, v_bits, dtype="bf16"):
    if dtype != "f32":
        return ko.attention_fp64(q_bits, k_bits, v_bits, dtype)
    hi = lambda b: (np.asarray(b, np.uint32) >> 16).astype(np.uint16)
    return ko.attention_fp64(hi(q_bits), hi(k_bits), hi(v_bits), "bf16")


def _round_f32_truncates(x, dtype="bf16"):
    if dtype != "f32":
        return ko.round_to_elem(x, dtype)
    x = np.asarray(x, np.float64)
    r = x.astype(np.float32)
    over = np.abs(r.astype(np.float64)) > np.abs(x)
    return np.where(over, np.nextafter(r, np.float32(0)), r).astype(np.float32).view(np.uint32)


def _round_truncates(x, dtype="bf16"):
    if dtype == "f16":
        return ko.round_to_elem(x, dtype)
    return (np.asarray(x, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _round_via_f32(x, dtype="bf16"):
    if dtype == "f16":
        return ko.round_to_elem(x, dtype)
    return ko.round_to_elem(np.asarray(x, np.float64).astype(np.float32).astype(np.float64), dtype)


def _round_ties_away(x, dtype="bf16"):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.trunc(m * (256.0 if dtype == "bf16" else 2048.0) + np.copysign(0.5, m))
    r = r * np.exp2(e.astype(np.float64) - (8.0 if dtype == "bf16" else 11.0))
    if dtype == "f16":
        return r.astype(np.float16).view(np.uint16)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _pins_fail(mutant, pins):
    for pin in pins:
        try:
            pin(mutant)
        except AssertionError:
            return True
    return False


ALL_PINS = [pin_worked_example, pin_special_closed_forms, pin_visible_set, pin_sdpa, pin_bruteforce,
            pin_softmax_invariants, pin_paged_equals_dense, pin_scale_phase, pin_rollback, pin_f16_inputs,
            pin_lse_base2, pin_f32_inputs, pin_round_to_f32, pin_round_to_elem, pin_rope_known_rotations, pin_rope_complex,
            pin_rope_norm_and_relative_position]


@pytest.mark.parametrize("mutant", [
    _Mutant(attention_fp64=_no_scale),
    _Mutant(attention_fp64=_values_are_keys),
    _Mutant(attention_fp64=_sum_over_queries),
    _Mutant(AllocatorReplay=_OffByOneWindow),
    _Mutant(AllocatorReplay=_SpecialsFirst),
    _Mutant(AllocatorReplay=_LastPageZeroWhenFull),
    _Mutant(AllocatorReplay=_ScaleEvicted),
    _Mutant(AllocatorReplay=_LifoSpecialReuse),
    _Mutant(AllocatorReplay=_OneFramePerStep),
    _Mutant(AllocatorReplay=_RollbackKeepsHeldBack),
    _Mutant(attention_fp64=_f16_read_as_bf16),
    _Mutant(lse_base2_fp64=_lse_natural_log),
    _Mutant(lse_base2_fp64=_lse_max_only),
    _Mutant(lse_base2_fp64=_lse_unscaled),
    _Mutant(rope_rotate_fp64=_rope_sign_slip),
    _Mutant(rope_rotate_fp64=_rope_dropped_term),
    _Mutant(rope_rotate_fp64=_rope_rotate_half),
    _Mutant(rope_rotate_fp64=_rope_inverse),
    _Mutant(round_to_elem=_round_truncates),
    _Mutant(round_to_elem=_round_via_f32),
    _Mutant(round_to_elem=_round_ties_away),
    _Mutant(attention_fp64=_f32_read_as_bf16),
    _Mutant(round_to_elem=_round_f32_truncates),
], ids=["no_scale", "values_are_keys", "wrong_softmax_axis", "window_off_by_one", "specials_first",
        "last_page_zero", "scale_evicted", "special_count_drift", "one_frame_per_step", "rollback_no_refill",
        "f16_read_as_bf16", "lse_natural_log", "lse_max_only", "lse_unscaled", "rope_sign_slip",
        "rope_dropped_term", "rope_rotate_half", "rope_inverse", "round_truncates", "round_via_f32",
        "round_ties_away", "f32_read_as_bf16", "round_f32_truncates"])
def test_planted_mistake_is_caught(mutant):
    # OracleStream inside the mutant must use the mutant's allocator
    class _Stream(ko.OracleStream):
        def __init__(self, cfg, blocks=(0,), free_patch_order=None, free_special_order=None):
            self.cfg = cfg
            self.alloc = mutant.AllocatorReplay(cfg, free_patch_order, free_special_order)
            self.pools = {b: ko.SimulatedPool(cfg) for b in blocks}

        def attend(self, plan, block, q_bits):
            qo = plan["qo_indptr"]
            outs = []
            for i in range(len(plan["last_page_len"])):
                k, v = mutant.gather_paged(self.cfg, self.pools[block], plan, i)
                outs.append(mutant.attention_fp64(q_bits[qo[i]:qo[i + 1]], k, v, self.cfg.dtype))
            return np.concatenate(outs)
    mutant.OracleStream = _Stream
    assert _pins_fail(mutant, ALL_PINS)
