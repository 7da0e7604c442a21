"""The fused append (kvc_run_append, KVC_OPT_FUSED_APPEND): a block's appends
of the step's frames and its attention in one attention launch that reads
the step's own rows from the caller's k and v, and one merge launch that also
copies them into the pool ([p5] "How Paged KV Cache Attention Achieves Stable
Inference in Ling-Bot-Map" §Frame Appending Without Dispatch Overhead).  The
result must be the separate path's, bit for bit, on the same plan (the plan
is the same either way: only where the own rows are read from differs);
within the 16-bit bounds of tests/stream_harness.py against the oracle; and
the pools must equal the oracle's bit for bit afterwards.  Where the fused
launch does not apply (16x16 kernel, no split) the call launches the appends
and the run instead, with the same guarantees."""
import dataclasses

import numpy as np
import pytest

import kvc_synth as syn
from tests.stream_harness import Harness, check_close

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(msg):
    print(msg, flush=True)


def _lockstep(wl, checks, S=1, blocks=2, opts=None, dtype="bf16"):
    """A fused and a separate-path harness over the same inputs; at the
    checked steps both run, outputs are compared bitwise and with the
    oracle."""
    import paged_kv_cache_kvc_amd as kvc
    o = {kvc.KVC_OPT_FUSED_APPEND: 1, **(opts or {})}
    hf = Harness(wl, num_blocks=blocks, max_frames_per_step=S, oracle_blocks=tuple(range(blocks)), fused=True,
                 options=opts)
    hs = Harness(wl, num_blocks=blocks, max_frames_per_step=S, oracle_blocks=(), options=o)
    last = None
    for t in range(max(wl.frames) - (S - 1)):
        nfr = {0: S} if t == 0 and S > 1 else None
        run = t in checks
        rf = hf.step(run=run, check=run, nframes=nfr)
        rs = hs.step(run=run, nframes=nfr)
        if run:
            for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr", "n_splits"):
                assert np.array_equal(rf["gpu_plan"][k], rs["gpu_plan"][k]), k
                if k != "n_splits":
                    assert np.array_equal(rf["gpu_plan"][k], rf["ora_plan"][k]), k
            for b in range(blocks):
                assert np.array_equal(rf["out_bits"][b], rs["out_bits"][b]), f"step {t} block {b}: fused != separate"
                st = check_close(rf["out_bits"][b], rf["ref"][b], dtype=dtype)
            log(f"{wl.name} step {t}: splits {rf['gpu_plan']['n_splits']} shape {hf.gpu.get_plan_shape()} {st}")
            last = rf
    for b in range(blocks):
        assert np.array_equal(hf.pool_bits(b), hf.ora.pools[b].data), f"pool {b}"
        assert np.array_equal(hs.pool_bits(b), hf.ora.pools[b].data), f"separate pool {b}"
    return hf, last


def test_fused_scale_step_and_streaming_d64():
    """H=4, D=64 over 80 frames: the 8-frame scale step, the first single
    frame, split steady states; two block pools."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(80,))
    hf, res = _lockstep(wl, {0, 1, 30, 72}, S=wl.scale_frames)
    assert max(res["gpu_plan"]["n_splits"]) > 1


def test_fused_tiny_every_step_and_specials_mid_frame():
    """D=32: the tiny stream at every step (a special unit cut where the
    step's specials start), and a frame whose 5 specials sit at rows 17..21
    of 45 (the patch units of the own frame cut at the special rows)."""
    _need_gpu()
    wl = syn.WORKLOADS["tiny"]
    _lockstep(wl, set(range(max(wl.frames))))
    mid = syn.Workload("mid_specials", 1, 2, 32, 40, 5, 64, 2, 6, (30,), 31,
                       max_patch_pages=2 + 6 + 1, max_special_pages=8, special_row_offset=17)
    _lockstep(mid, {0, 1, 2, 7, 29}, S=2)


def test_fused_two_streams_f16():
    """Two streams (one joining later) at D=64 in float16: each work item
    reads its own stream's k and v."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(40, 70), dtype="f16",
                             max_patch_pages=2 * (8 + 64 + 1))
    _lockstep(wl, {0, 31, 45, 69}, blocks=1, dtype="f16")


def test_fused_call_falls_back_where_it_cannot_fuse():
    """No split (KVC_OPT_MAX_SPLITS 1) and the 16x16 kernel (D=128): the call
    launches the appends and the run; same results."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(20,))
    _lockstep(wl, {0, 19}, blocks=1, opts={kvc.KVC_OPT_MAX_SPLITS: 1})
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(20,), head_dim=128)
    _lockstep(wl, {0, 19}, blocks=1)


def test_fused_call_order_errors():
    """A deferred append must be completed by kvc_run_append: kvc_run on
    that block, a new step, a rollback and switching the option off are
    refused while it is pending; kvc_run_append needs a fused plan and
    refuses a block already appended with its rows."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = syn.WORKLOADS["tiny"]
    T, H, D = wl.tokens_per_frame, wl.num_heads, wl.head_dim
    from tests.stream_harness import cfg_args
    c = kvc.PagedKVCache(kvc.make_config(**cfg_args(wl, 2)), device="cuda")
    k = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros_like(k)
    with pytest.raises(kvc.KvcError):
        c.append_frames(0, num_frames=1, defer=True)          # option off
    c.set_option(kvc.KVC_OPT_DEFER_EVICTION, 1)
    c.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    c.append_frames(0, num_frames=1, defer=True)
    c.plan()
    with pytest.raises(kvc.KvcError):
        c.compute_attention(0, q)                             # deferred: kvc_run refused
    with pytest.raises(kvc.KvcError):
        c.set_option(kvc.KVC_OPT_FUSED_APPEND, 0)
    with pytest.raises(kvc.KvcError):
        c.rollback_frame(0)
    with pytest.raises(kvc.KvcError):
        c.append_frames(0, num_frames=1, defer=True)          # new step while pending
    c.append_run(0, {0: k}, {0: k}, q)
    c.append_frame(1, k, k)
    with pytest.raises(kvc.KvcError):
        c.append_run(1, {0: k}, {0: k}, q)                    # block 1 already has its rows
    c.compute_attention(1, q)
    torch.cuda.synchronize()
    # a plan built before the option was set is not fused
    c2 = kvc.PagedKVCache(kvc.make_config(**cfg_args(wl, 1)), device="cuda")
    c2.append_frame(0, k, k)
    c2.plan()
    c2.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    with pytest.raises(kvc.KvcError):
        c2.append_run(0, {0: k}, {0: k}, q)


def test_fused_base_full_size():
    """The benchmark's step at its full shape: H=16, D=64, 262 tokens per
    frame, 200 frames, two block pools, every step through kvc_run_append
    where it runs; checked at ragged and steady-state steps against the
    oracle (the launch configuration bench.py times: 256 work-groups of
    the 32x32 kernel with tails, 16 splits), pools bit-exact at the end."""
    _need_gpu()
    wl = syn.WORKLOADS["base"]
    checks = {0, 1, 72, 150, 199}
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1), fused=True)
    for t in range(max(wl.frames)):
        res = h.step(run=t in checks, check=t in checks)
        if t in checks:
            for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr"):
                assert np.array_equal(res["gpu_plan"][k], res["ora_plan"][k]), k
            for b in (0, 1):
                st = check_close(res["out_bits"][b], res["ref"][b])
            log(f"fused base step {t}: splits {res['gpu_plan']['n_splits']} shape {h.gpu.get_plan_shape()} {st}")
    assert h.gpu.get_plan_shape() == {"work_items": 256, "group_rows": 272}
    assert list(res["gpu_plan"]["n_splits"]) == [16]
    for b in (0, 1):
        assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data)
