"""The bfloat16 32x32 kernel's exact path works from the packed
probabilities (an exact integer rebase) and falls back to a second pass over
the split with the scores when they cannot stand in: a probability that
overflowed, or a first stage whose largest probability is far below the
reference (terms may have underflowed).  Planted keys force both cases
([p1] "How FlashInfer KV Cache Attention Accelerates Streaming 3D
Reconstruction Over SDPA" §Efficient Attention Masking and Padding: the
softmax is over every valid token, however the scores are spread); the
result must still be the oracle's within the 16-bit bounds, on split and
unsplit plans, with and without the fused append."""
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


def _planted(h, hi_frames, lo_frames, amp):
    """Queries get +amp along dimension 0 of every head; keys of hi_frames
    +amp (scores near +amp^2 / sqrt(D): far above every earlier stage), keys
    of lo_frames -amp (scores near -amp^2 / sqrt(D): far below)."""
    orig = h._frame

    def frame(s, f, b, which):
        bits = orig(s, f, b, which)
        if which == "v" or (which == "k" and f not in hi_frames and f not in lo_frames):
            return bits
        dt = h.wl.dtype
        x = syn.bits_to_f32(bits, dt).astype(np.float32)   # [T, H, D]
        sign = 1.0 if which == "q" or f in hi_frames else -1.0
        x[..., 0] += np.float32(sign * amp)
        return syn.f32_to_bits(x, dt)

    h._frame = frame


@pytest.mark.parametrize("case", ["bf16", "bf16-fused", "f16", "d128"])
def test_planted_overflow_and_underflow(case):
    """Frames 0-3 (the start of the table: the first stages of the first
    splits) hold keys far below the queries' scores elsewhere, frames 20 and
    33 keys far above; with amp = 40 at D=64 the scores are about +-200 (in
    base-2 units +-290): the optimistic probabilities overflow or vanish.
    bfloat16 with and without the fused append, float16 (its probabilities
    saturate instead of overflowing), and D=128 (the 16x16 kernel); split
    and unsplit plans."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    dtype = "f16" if case == "f16" else "bf16"
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(40,), dtype=dtype,
                             head_dim=128 if case == "d128" else 64)
    for opts in ({}, {kvc.KVC_OPT_MAX_SPLITS: 1}):
        h = Harness(wl, fused=case == "bf16-fused", options=opts)
        _planted(h, hi_frames={20, 33}, lo_frames={0, 1, 2, 3}, amp=40.0)
        for t in range(max(wl.frames)):
            res = h.step(run=t in (10, 25, 39), check=t in (10, 25, 39))
            if t in (10, 25, 39):
                st = check_close(res["out_bits"][0], res["ref"][0], dtype=dtype)
                log(f"{case} opts={opts} step {t}: splits {res['gpu_plan']['n_splits']} {st}")
        assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_planted_underflow_everywhere():
    """Every key far below the queries (scores near -200): every first
    stage's probabilities vanish against the initial reference; the second
    pass must give the plain softmax of those scores."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(24,))
    h = Harness(wl)
    _planted(h, hi_frames=set(), lo_frames=set(range(24)), amp=40.0)
    for t in range(max(wl.frames)):
        res = h.step(run=t in (0, 23), check=t in (0, 23))
        if t in (0, 23):
            st = check_close(res["out_bits"][0], res["ref"][0])
            log(f"all keys low, step {t}: splits {res['gpu_plan']['n_splits']} {st}")
