"""head_dim 64 served by either attention kernel: the 32x32 one (groups of
eight 32-row tiles, one work-group per CU) and the 16x16 one (groups of eight
16-row tiles, two work-groups per CU), chosen per plan by the planner or
fixed with KVC_OPT_QUERY_TILE.  The same attention ([p3] "How FlashInfer's
Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference",
§Dual-Stream Attention) must come out of both within the 16-bit bounds of
tests/stream_harness.py, on split and unsplit plans, ragged first steps, the
multi-frame scale step and both 16-bit element types; pools bit-exact."""
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


def _plans_equal(res):
    g, r = res["gpu_plan"], res["ora_plan"]
    for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr"):
        assert np.array_equal(g[k], r[k]), k


@pytest.mark.parametrize("tile", [16, 32])
def test_d64_forced_tile_steps_and_scale(tile):
    """H=4 over 80 frames with the kernel fixed: the 8-frame scale step, the
    first single-frame step, a split steady state and sharpened queries."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(80,))
    S = wl.scale_frames
    h = Harness(wl, num_blocks=2, max_frames_per_step=S, oracle_blocks=(0, 1),
                options={kvc.KVC_OPT_QUERY_TILE: tile})
    rows = 128 if tile == 16 else 256
    res = h.step(check=True, nframes={0: S})
    _plans_equal(res)
    assert h.gpu.get_plan_shape()["group_rows"] in (rows, rows + 16)
    for b in (0, 1):
        st = check_close(res["out_bits"][b], res["ref"][b])
    log(f"tile {tile} scale step: splits {res['gpu_plan']['n_splits']} {st}")
    last = max(wl.frames) - S
    for t in range(1, last + 1):
        res = h.step(run=t in (1, last), check=t in (1, last))
        if t in (1, last):
            _plans_equal(res)
            assert h.gpu.get_plan_shape()["group_rows"] in (rows, rows + 16)
            for b in (0, 1):
                st = check_close(res["out_bits"][b], res["ref"][b])
            log(f"tile {tile} step {t}: splits {res['gpu_plan']['n_splits']} {st}")
    assert max(res["gpu_plan"]["n_splits"]) > 1
    q3 = syn.f32_to_bf16_bits(syn.bf16_bits_to_f32(res["q_bits"][0]) * 3.0)
    out = h.gpu.compute_attention(0, h.to_dev(q3))
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    st3 = check_close(bits, h.ora.attend(res["ora_plan"], 0, q3))
    log(f"tile {tile} sharpened: {st3}")
    for b in (0, 1):
        assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data)


def test_d64_tiles16_f16_and_unsplit():
    """float16 pools on the 16x16 kernel at head_dim 64, with and without
    split-KV."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(40,), dtype="f16")
    for opts in ({kvc.KVC_OPT_QUERY_TILE: 16}, {kvc.KVC_OPT_QUERY_TILE: 16, kvc.KVC_OPT_MAX_SPLITS: 1}):
        h = Harness(wl, options=opts)
        for t in range(max(wl.frames)):
            res = h.step(run=t in (0, 39), check=t in (0, 39))
            if t in (0, 39):
                _plans_equal(res)
                assert h.gpu.get_plan_shape()["group_rows"] == 128
                st = check_close(res["out_bits"][0], res["ref"][0], dtype="f16")
                log(f"f16 tile 16 {opts} step {t}: splits {res['gpu_plan']['n_splits']} {st}")
        assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_scale_step_32_heads_planner_choice():
    """The 8-frame scale step over 32 heads at D=64 (2096 queries over 2096
    tokens per head) on the planner's own choice, the 16x16 kernel: the
    32x32 kernel's 288 groups would leave 32 CUs a second one, while the 544
    groups of 128 rows run at most three to a CU, two of them resident
    together."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=32, frames=(12,))
    S = wl.scale_frames
    # the planner's target on a 256-CU device, fixed so the plan's shape is known
    h = Harness(wl, max_frames_per_step=S, options={kvc.KVC_OPT_TARGET_WORKGROUPS: 256})
    res = h.step(check=True, nframes={0: S})
    _plans_equal(res)
    shape = h.gpu.get_plan_shape()
    log(f"scale step plan: {shape}, splits {res['gpu_plan']['n_splits']}")
    assert shape == {"work_items": 544, "group_rows": 128}
    st = check_close(res["out_bits"][0], res["ref"][0])
    log(f"scale step H=32, planner choice: {st}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)
