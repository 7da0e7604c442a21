"""Parity of the HIP path (through the C-ABI) with the CPU oracle on MI355X.

Page tables and last-page lengths must be bit-exact, the pools bit-exact with
the oracle's simulated pools (valid and pad slots), and the attention output
within |o - o_ref| <= 1e-2 + 1e-2 |o_ref| of the float64 oracle.  Inputs are
the seeded synthetic streams of kvc_synth at the workload shapes; checked
sizes span many 64-token KV stages, several query tiles and ragged tails."""
import numpy as np
import pytest

import kvc_synth as syn
from tests.stream_harness import Harness, check_close, check_split_matches_unsplit, final_visible

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def compare_plan(res):
    g, r = res["gpu_plan"], res["ora_plan"]
    for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr"):
        assert np.array_equal(g[k], r[k]), k


def log(msg):
    print(msg, flush=True)


def test_tiny_stream_every_step_two_blocks():
    _need_gpu()
    wl = syn.WORKLOADS["tiny"]
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1))
    for t in range(max(wl.frames)):
        res = h.step(check=True)
        compare_plan(res)
        for b in (0, 1):
            st = check_close(res["out_bits"][b], res["ref"][b])
        for b in (0, 1):
            assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data), f"pool block {b} step {t}"
    log(f"tiny ok {st}")


def test_tiny_specials_first_and_no_split():
    _need_gpu()
    import dataclasses
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["tiny"], special_row_offset=0)
    h = Harness(wl, options={kvc.KVC_OPT_MAX_SPLITS: 1})
    for t in range(max(wl.frames)):
        res = h.step(check=True)
        assert res["gpu_plan"]["n_splits"][0] == 1
        check_close(res["out_bits"][0], res["ref"][0])
        assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def _base_small(H=4, frames=90):
    import dataclasses
    return dataclasses.replace(syn.WORKLOADS["base"], num_heads=H, frames=(frames,))


def test_split_equals_no_split_and_sharpened_queries():
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = _base_small(H=4, frames=80)
    outs = []
    for opts in ({}, {kvc.KVC_OPT_MAX_SPLITS: 1}):
        h = Harness(wl, q_scale=3.0, options=opts)
        for t in range(max(wl.frames)):
            res = h.step(run=t in (0, 40, 79), check=t in (0, 79))
            if t in (0, 79):
                st = check_close(res["out_bits"][0], res["ref"][0])
        outs.append(res["out_bits"][0])
        log(f"opts {opts} splits {res['gpu_plan']['n_splits']} {st}")
    a = syn.bf16_bits_to_f32(outs[0])
    b = syn.bf16_bits_to_f32(outs[1])
    log(f"split vs unsplit: max diff / std {check_split_matches_unsplit(a, b)}")


def test_page_permutation_invariance_bitwise():
    _need_gpu()
    wl = _base_small(H=2, frames=100)
    bits = []
    for orders in (None, 11):
        from tests.stream_harness import free_orders
        h = Harness(wl, orders=free_orders(wl, orders) if orders else (None, None))
        for t in range(max(wl.frames)):
            res = h.step(run=t == max(wl.frames) - 1)
        bits.append(res["out_bits"][0])
        if orders:
            assert not np.array_equal(res["gpu_plan"]["kv_indices"], first_indices)
        first_indices = res["gpu_plan"]["kv_indices"]
    assert np.array_equal(bits[0], bits[1])


def test_base_full_size_parity_and_pool():
    """The 256-patch, 64-frame-window workload at full H=16, D=64 over its
    200 frames, checked at ragged and steady-state steps, two block pools;
    at the checked steps the same plan also runs sharpened queries (q x 3,
    a peaked softmax whose output spread is far above the tolerance)."""
    _need_gpu()
    wl = syn.WORKLOADS["base"]
    checks = {0, 1, 71, 72, 150, 199}
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1))
    for t in range(max(wl.frames)):
        res = h.step(run=t in checks, check=t in checks)
        if t in checks:
            compare_plan(res)
            for b in (0, 1):
                st = check_close(res["out_bits"][b], res["ref"][b])
            log(f"base step {t}: splits {res['gpu_plan']['n_splits']} {st}")
            if t in (72, 199):
                q3 = h._frame(0, t, 0, "q").copy()
                q3 = syn.f32_to_bf16_bits(syn.bf16_bits_to_f32(q3) * 3.0)
                out = h.gpu.compute_attention(0, h.to_dev(q3))
                bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
                st3 = check_close(bits, h.ora.attend(res["ora_plan"], 0, q3))
                log(f"base step {t} sharpened q x 3: {st3}")
    # the launch timed by bench.py
    log(f"plan shape {h.gpu.get_plan_shape()}")
    for b in (0, 1):
        assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data)


def test_run_twice_bitwise_and_profile():
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = _base_small(H=4, frames=30)
    h = Harness(wl, options={kvc.KVC_OPT_PROFILE: 1})
    for t in range(30):
        res = h.step(run=True)
    q = np.concatenate([h._frame(0, 29, 0, "q")])
    qd = h.to_dev(q)
    o1 = h.gpu.compute_attention(0, qd)
    o2 = h.gpu.compute_attention(0, qd)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ms, n = h.gpu.profile_read(kvc.KVC_KERNEL_ATTENTION)
    assert n == 32 and ms > 0
    ms, n = h.gpu.profile_read(kvc.KVC_KERNEL_APPEND)
    assert n == 30


def test_r518_padded_pages_and_poisoned_slots():
    """999 patches in 1024-token pages (pad slots excluded by length) over
    500 frames; then NaN/huge poison in every pad slot and beyond the tail
    length must leave the output bit-identical."""
    _need_gpu()
    wl = syn.WORKLOADS["r518"]
    F = max(wl.frames)
    checks = {9, F - 1}
    real = final_visible(wl, 0, extra_steps=checks)
    h = Harness(wl, real_patch=lambda s, f: f in real)
    for t in range(F):
        res = h.step(run=t in checks, check=t in checks)
        if t in checks:
            compare_plan(res)
            st = check_close(res["out_bits"][0], res["ref"][0])
            log(f"r518 step {t}: splits {res['gpu_plan']['n_splits']} {st}")
    # the full-size step runs the 32x32 kernel without a tail (4 groups of 8 tiles)
    assert h.gpu.get_plan_shape() == {"work_items": 256, "group_rows": 256}
    before = res["out_bits"][0]
    plan = res["gpu_plan"]
    pool = h.gpu.pools[0]
    P, pg = wl.patch_tokens, wl.page_size
    idx = plan["kv_indices"]
    npatch = plan["n_patch_pages"][0]
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    for j, page in enumerate(idx):
        if j < npatch:
            pool[int(page), :, P:] = nan
        elif j == len(idx) - 1:
            pool[int(page), :, plan["last_page_len"][0]:] = 3.0e38
    # rerun the last step's attention on the same plan
    q = h._frame(0, F - 1, 0, "q")
    out = h.gpu.compute_attention(0, h.to_dev(q))
    after = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(before, after)


def test_long_stream_constant_footprint():
    """10,000 frames (60,000 special tokens): output at the last step, and no
    device allocation by the library while streaming."""
    _need_gpu()
    wl = syn.WORKLOADS["long"]
    F = max(wl.frames)
    real = final_visible(wl, 0)
    h = Harness(wl, real_patch=lambda s, f: f in real)
    # The device's free memory (mem_get_info sees every allocation on the
    # device, the library's included, not only torch's) must not move while
    # the stream runs: the first 100 steps settle the runtime, then the
    # reading is taken every 2000 frames.
    free0 = None
    for t in range(F - 1):
        h.step(run=False)
        if t == 100 or (t > 100 and t % 2000 == 0):
            torch.cuda.synchronize()
            free, _ = torch.cuda.mem_get_info()
            if free0 is None:
                free0 = free
            assert free == free0, f"device free memory moved by {free0 - free} bytes after {t} frames"
            log(f"long: {t} frames, device free memory unchanged")
    res = h.step(run=True, check=True)
    compare_plan(res)
    st = check_close(res["out_bits"][0], res["ref"][0])
    log(f"long final: splits {res['gpu_plan']['n_splits']} {st}")
    stats = h.gpu.get_cache_stats()
    assert stats["special_tokens"] == 60000 and stats["special_pages"] == 235 and stats["live_pages"] == 64


def test_fragmented_four_streams():
    """Four streams (50/400/1500/4000 frames) in one plan/run, H=8, D=128,
    both free lists shuffled from the seed."""
    _need_gpu()
    wl = syn.WORKLOADS["frag"]
    total = max(wl.frames)
    reals = [final_visible(wl, s) for s in range(wl.num_streams)]
    h = Harness(wl, real_patch=lambda s, f: f in reals[s])
    for t in range(total - 1):
        h.step(run=False)
    res = h.step(run=True, check=True)
    compare_plan(res)
    st = check_close(res["out_bits"][0], res["ref"][0])
    log(f"frag: splits {res['gpu_plan']['n_splits']} {st}")


def test_scale_phase_multi_frame_prefill():
    """[p2] §Frame Processing Loop: the first S frames in one step (S*T
    queries attending every token of those frames), then single-frame
    streaming.  Outputs within tolerance, plans and pool bit-exact."""
    _need_gpu()
    wl = _base_small(H=4, frames=90)
    S, T = wl.scale_frames, wl.tokens_per_frame
    h = Harness(wl, num_blocks=2, max_frames_per_step=S, oracle_blocks=(0, 1))
    res = h.step(check=True, nframes={0: S})
    compare_plan(res)
    assert list(res["gpu_plan"]["qo_indptr"]) == [0, S * T]
    for b in (0, 1):
        st = check_close(res["out_bits"][b], res["ref"][b])
        log(f"scale-phase step block {b}: splits {res['gpu_plan']['n_splits']} {st}")
    last = max(wl.frames) - S
    for t in range(1, last + 1):
        res = h.step(run=t in (1, 40, last), check=t in (1, last))
        compare_plan(res)
        if "ref" in res:
            check_close(res["out_bits"][0], res["ref"][0])
    assert h.frame_of[0] == max(wl.frames)
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_scale_phase_full_heads():
    """The 8-frame scale step at the full H=16, D=64 shape on the 32x32
    kernel: 2096 queries over 2096 tokens in 144 work-groups (9 query groups
    of 8 tiles of 32 rows per head, one split: a second split would need a
    second round of work-groups and a merge); output against the oracle,
    pool bit-exact."""
    _need_gpu()
    import dataclasses
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["base"], frames=(12,))
    S = wl.scale_frames
    h = Harness(wl, max_frames_per_step=S, options={kvc.KVC_OPT_QUERY_TILE: 32})
    res = h.step(check=True, nframes={0: S})
    compare_plan(res)
    assert list(res["gpu_plan"]["n_splits"]) == [1]
    assert h.gpu.get_plan_shape()["work_items"] == 144
    st = check_close(res["out_bits"][0], res["ref"][0])
    log(f"scale step H=16: {st}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_deferred_eviction_with_rollbacks():
    """Frame rollback with deferred eviction ([p2] §Scale Frames vs Sliding
    Window): every fourth frame is undone after its step; attention stays
    within tolerance of the oracle replaying the same rules, the stale plan
    cannot be run after a rollback, and the pool matches bit-exactly."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = _base_small(H=4, frames=100)
    h = Harness(wl)
    h.gpu.set_option(kvc.KVC_OPT_DEFER_EVICTION, 1)
    h.ora.alloc.defer_eviction = True
    rolled = 0
    for t in range(max(wl.frames)):
        res = h.step(run=t % 10 == 9 or t % 4 == 2, check=t % 20 == 19 or t in (2, 78))
        compare_plan(res)
        if "ref" in res:
            st = check_close(res["out_bits"][0], res["ref"][0])
            log(f"step {t} frames {h.gpu.get_cache_stats()['frame_count']} {st}")
        if t % 4 == 2 and t < 90:
            h.rollback(0)
            rolled += 1
            q = h.torch.zeros((wl.tokens_per_frame, wl.num_heads, wl.head_dim), dtype=h.torch.bfloat16,
                              device=h.device)
            with pytest.raises(kvc.KvcError) as e:
                h.gpu.compute_attention(0, q)
            assert e.value.status == kvc.KVC_ERR_STATE
    assert h.gpu.get_cache_stats()["frame_count"] == max(wl.frames) - rolled
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_f16_pools_d32_d64_d128():
    """IEEE-half pools and inputs ([p3] §Precision and Hardware Utilization:
    the paged kernels take fp16 as well as bf16): the tiny stream at every
    step (D=32, two blocks, pools bit-exact), the base shape with sharpened
    queries split and unsplit (D=64), and D=128 over a shorter stream, each
    against the oracle on the same f16 inputs."""
    _need_gpu()
    import dataclasses
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["tiny"], dtype="f16")
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1))
    for t in range(max(wl.frames)):
        res = h.step(check=True)
        compare_plan(res)
        for b in (0, 1):
            st = check_close(res["out_bits"][b], res["ref"][b], dtype="f16")
            assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data), f"pool block {b} step {t}"
    log(f"f16 tiny ok {st}")
    wl = dataclasses.replace(_base_small(H=4, frames=80), dtype="f16")
    outs = []
    for opts in ({}, {kvc.KVC_OPT_MAX_SPLITS: 1}):
        h = Harness(wl, q_scale=3.0, options=opts)
        for t in range(max(wl.frames)):
            res = h.step(run=t in (0, 79), check=t in (0, 79))
            if t in (0, 79):
                st = check_close(res["out_bits"][0], res["ref"][0], dtype="f16")
        outs.append(syn.bits_to_f32(res["out_bits"][0], "f16"))
        log(f"f16 base opts {opts} splits {res['gpu_plan']['n_splits']} {st}")
        assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)
    check_split_matches_unsplit(outs[0], outs[1])
    wl = dataclasses.replace(_base_small(H=2, frames=75), head_dim=128, dtype="f16")
    h = Harness(wl)
    for t in range(max(wl.frames)):
        res = h.step(run=t in (3, 74), check=t in (3, 74))
        if t in (3, 74):
            compare_plan(res)
            st = check_close(res["out_bits"][0], res["ref"][0], dtype="f16")
            log(f"f16 D=128 step {t} splits {res['gpu_plan']['n_splits']} {st}")


@pytest.mark.parametrize("name", ["no_specials", "max_specials", "one_token", "steps_of_64"])
def test_degenerate_shapes(name):
    """Frames without special tokens, 64 special tokens per frame over four
    pages, one-token frames (one head, D=128, one-slot pages), and a first
    step of 64 frames: page tables, pools (bit-exact) and attention against
    the oracle at every step."""
    _need_gpu()
    from tests.stream_harness import edge_workloads
    wl = edge_workloads()[name]
    multi = 64 if name == "steps_of_64" else 1
    h = Harness(wl, max_frames_per_step=multi)
    done = 0
    while done < max(wl.frames):
        nf = multi if done == 0 else 1
        res = h.step(check=True, nframes={0: nf})
        compare_plan(res)
        st = check_close(res["out_bits"][0], res["ref"][0])
        assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data), f"pool after {done} frames"
        done += nf
    log(f"{name}: {done} frames, splits {res['gpu_plan']['n_splits']} {st}")
