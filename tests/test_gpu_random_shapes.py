"""Seeded random shapes against the oracle.

Each case draws the cache's geometry and the planner's options: head count,
head_dim (32, 64, 128), element type (bf16, f16, f32), patch tokens per frame and
the page size above them, special tokens per frame and the rows they take in
the frame, scale frames, window, one to three streams (later ones joining
late), shuffled free lists, a multi-frame first step, the split cap, the
work-group target, the head_dim 64 kernel and the fused append.  The frame
stream is run through the library and the oracle side by side ([p3] "How
FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in Streaming
Inference" §Dual-Stream Attention; [p1] "How FlashInfer KV Cache Attention
Accelerates Streaming 3D Reconstruction Over SDPA" §Two-Stream Design for
Token Types): at the checked steps the plan equals the oracle's and the
output is within the element type's bounds of tests/stream_harness.py; at
the end the pools equal the oracle's bit for bit.  The draws are bounded so
that a case runs in a few seconds."""
import dataclasses

import numpy as np
import pytest

import kvc_synth as syn
from tests.stream_harness import Harness, check_close

torch = pytest.importorskip("torch")

CASES = 48


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_case(i: int):
    """The workload, options, harness flags and checked steps of case i
    (numpy's PCG64 seeded with 7100 + i)."""
    import paged_kv_cache_kvc_amd as kvc
    rng = np.random.default_rng(7100 + i)
    D = int(rng.choice([32, 64, 128]))
    H = int(rng.choice([1, 2, 3, 4] if D == 128 else [1, 2, 3, 4, 6, 8]))
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.4, 0.4, 0.2]))
    P = int(rng.integers(1, 261))
    n_s = int(rng.choice([0, 1, 5, int(rng.integers(1, 17))]))
    # (at least 4 slots: one frame's specials then span at most 8 pages)
    page = max(4, int(rng.choice([P, -(-P // 16) * 16, max(P, 256)])))
    row_off = P if rng.random() < 0.6 else int(rng.integers(0, P + 1))
    S = int(rng.integers(0, 5))
    W = int(rng.integers(1, 9))
    nstreams = int(rng.choice([1, 1, 2, 3]))
    frames = tuple(int(rng.integers(max(2, S + W + 2), S + W + 10)) if k == 0 else int(rng.integers(2, S + W + 6))
                   for k in range(nstreams))
    multi = nstreams == 1 and S >= 2 and rng.random() < 0.5
    max_sp = sum(-(-f * n_s // page) + 1 for f in frames) if n_s else 0
    wl = syn.Workload(f"random{i}", 2, H, D, P, n_s, page, S, W, frames, 500 + i,
                      max_patch_pages=nstreams * (S + W + 1) + int(rng.integers(0, 3)),
                      max_special_pages=max_sp, shuffle_free_lists=bool(rng.random() < 0.5),
                      special_row_offset=row_off, dtype=dtype)
    opts = {}
    if rng.random() < 0.4:
        opts[kvc.KVC_OPT_MAX_SPLITS] = int(rng.choice([1, 2, 3, 5]))
    if rng.random() < 0.4:
        opts[kvc.KVC_OPT_TARGET_WORKGROUPS] = int(rng.choice([8, 64, 256, 1024]))
    if D == 64 and rng.random() < 0.5:
        opts[kvc.KVC_OPT_QUERY_TILE] = int(rng.choice([16, 32]))
    fused = bool(rng.random() < 0.5)
    nsteps = max(frames) - ((S - 1) if multi else 0)
    checks = {0, 1, nsteps - 1, int(rng.integers(2, max(3, nsteps - 1)))}
    return wl, opts, fused, multi, nsteps, checks


def test_draws_cover_the_options():
    """The case list reaches every element type, head_dim, several streams,
    the multi-frame step, specials inside the frame and the fused append."""
    import paged_kv_cache_kvc_amd as kvc
    seen = set()
    for i in range(CASES):
        wl, opts, fused, multi, _, _ = draw_case(i)
        seen |= {("D", wl.head_dim), ("dtype", wl.dtype), ("streams>1", wl.num_streams > 1), ("multi", multi),
                 ("fused", fused), ("mid", wl.row_offset < wl.patch_tokens and wl.num_special_tokens > 0),
                 ("tile", opts.get(kvc.KVC_OPT_QUERY_TILE, 0))}
    for want in (("D", 32), ("D", 64), ("D", 128), ("dtype", "bf16"), ("dtype", "f16"), ("dtype", "f32"),
                 ("streams>1", True),
                 ("multi", True), ("fused", True), ("fused", False), ("mid", True)):
        assert want in seen, want


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(CASES))
def test_random_shape(case):
    _need_gpu()
    wl, opts, fused, multi, nsteps, checks = draw_case(case)
    print(f"case {case}: {dataclasses.asdict(wl)} options {opts} fused {fused} multi {multi} checks {sorted(checks)}",
          flush=True)
    S = wl.scale_frames
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1), options=opts, fused=fused,
                max_frames_per_step=S if multi else 1)
    for t in range(nsteps):
        run = t in checks
        res = h.step(run=run, check=run, nframes={0: S} if multi and t == 0 else None)
        if run:
            for k in ("kv_indptr", "kv_indices", "last_page_len", "n_patch_pages", "qo_indptr"):
                assert np.array_equal(res["gpu_plan"][k], res["ora_plan"][k]), k
            for b in (0, 1):
                st = check_close(res["out_bits"][b], res["ref"][b], dtype=wl.dtype)
            print(f"  step {t}: splits {res['gpu_plan']['n_splits']} shape {h.gpu.get_plan_shape()} {st}", flush=True)
    for b in (0, 1):
        assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data), f"pool {b}"
