"""kvc_run_no_alloc, the variant of kvc_run for callers that cannot allocate
device memory (split partials in the library's static device scratch),
against kvc_run through the C-ABI: bit-identical outputs on the same plan,
within tolerance of the oracle, on two calls in a row with the second on a
smaller input (a second context, smaller shape, fewer splits), and refused
with KVC_ERR_CAPACITY when a plan's partials would not fit."""
import numpy as np
import pytest

import kvc_synth as syn
from tests.stream_harness import Harness, check_close

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_both(h, t, block=0):
    """kvc_run and kvc_run_no_alloc on the current plan of block `block`."""
    q = np.concatenate([h._frame(0, t, block, "q")])
    qd = h.to_dev(q)
    ref_out = h.gpu.compute_attention(block, qd)
    out = torch.empty_like(qd)
    h.gpu.compute_attention(block, qd, out=out, no_alloc=True)
    torch.cuda.synchronize()
    a = ref_out.view(torch.int16).cpu().numpy().view(np.uint16)
    b = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return q, a, b


def test_no_alloc_matches_run_twice_second_smaller():
    _need_gpu()
    import dataclasses
    import paged_kv_cache_kvc_amd as kvc
    # first call: base shape at H=8 over 80 frames (split KV)
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=8, frames=(80,))
    h = Harness(wl)
    for t in range(80):
        res = h.step(run=t == 79, check=t == 79)
    assert res["gpu_plan"]["n_splits"][0] > 1
    q, a, b = _run_both(h, 79)
    assert np.array_equal(a, b)
    check_close(b, h.ora.attend(res["ora_plan"], 0, q))
    print(f"no_alloc base: splits {res['gpu_plan']['n_splits']}", flush=True)
    # second call, smaller input: the tiny stream in a new context
    wl2 = syn.WORKLOADS["tiny"]
    h2 = Harness(wl2)
    for t in range(max(wl2.frames)):
        res2 = h2.step(run=False)
    q2, a2, b2 = _run_both(h2, max(wl2.frames) - 1)
    assert np.array_equal(a2, b2)
    check_close(b2, h2.ora.attend(res2["ora_plan"], 0, q2))
    print(f"no_alloc tiny: splits {res2['gpu_plan']['n_splits']}", flush=True)
    # and the first context again, after the smaller call overwrote the scratch
    q3, a3, b3 = _run_both(h, 79)
    assert np.array_equal(a3, b3) and np.array_equal(b3, b)


def test_no_alloc_refuses_partials_beyond_the_scratch():
    """A plan whose split partials exceed KVC_NO_ALLOC_SCRATCH_BYTES is refused
    before any launch (64 heads, D=128, 1005-row frames, 64 splits); kvc_run
    with the caller's workspace still runs it."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    cfg = kvc.make_config(1, 64, 128, 1005, 6, page_size=1024, scale_frames=1, sliding_window=4,
                          max_patch_pages=6, max_special_pages=1)
    cache = kvc.PagedKVCache(cfg, device="cuda")
    k = torch.zeros((1005, 64, 128), dtype=torch.bfloat16, device="cuda")
    # plan for far more work-groups than the device holds, so every unit of
    # the stream gets a split of its own (up to 64)
    cache.set_option(kvc.KVC_OPT_TARGET_WORKGROUPS, 1 << 16)
    cache.set_option(kvc.KVC_OPT_MAX_SPLITS, 64)
    for _ in range(5):
        cache.append_frame(0, k, k)
        cache.evict_frames()
        cache.plan()
    assert max(cache.get_plan()["n_splits"]) == 64
    out = torch.empty_like(k)
    with pytest.raises(kvc.KvcError) as e:
        cache.compute_attention(0, k, out=out, no_alloc=True)
    assert e.value.status == kvc.KVC_ERR_CAPACITY
    cache.compute_attention(0, k, out=out)
    torch.cuda.synchronize()
