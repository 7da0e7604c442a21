"""Float32 pools on the HIP path (the full-precision variant: [p3] "How
FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in Streaming
Inference", FAQ on fp32 precision; [p4] "FlashInfer Backend in LingBot-Map:
Accelerating Streaming Inference with Paged KV Cache" §Memory Management and
Debugging).  K, V, Q and O are float32; the attention kernel computes in
float32 throughout (float32 MFMA, probabilities not rounded), so its output
must agree with the float64 oracle to the float32 bounds of
tests/stream_harness.py (relative RMS 2^-16, max error 2^-12 of the output's
spread, elementwise 1e-5 + 1e-4 |ref|), far tighter than the 16-bit types.
Pools, with and without the rotary embedding, are bit-exact."""
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


def test_f32_tiny_every_step_two_blocks():
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["tiny"], dtype="f32")
    h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1))
    for t in range(max(wl.frames)):
        res = h.step(check=True)
        _plans_equal(res)
        assert list(res["gpu_plan"]["n_splits"]) == [1]
        for b in (0, 1):
            st = check_close(res["out_bits"][b], res["ref"][b], dtype="f32")
            assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data), f"pool block {b} step {t}"
    log(f"f32 tiny ok {st}")


def test_f32_d64_long_context_and_sharpened_queries():
    """D=64 over 80 frames (4 heads): ragged first step and a steady state of
    about 19.6k tokens, then the same plan with queries x 3 (a peaked
    softmax)."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(80,), dtype="f32")
    h = Harness(wl)
    last = max(wl.frames) - 1
    for t in range(max(wl.frames)):
        res = h.step(run=t in (0, last), check=t in (0, last))
        if t in (0, last):
            _plans_equal(res)
            st = check_close(res["out_bits"][0], res["ref"][0], dtype="f32")
            log(f"f32 D=64 step {t}: {st}")
    q3 = syn.f32_to_bits(syn.bits_to_f32(res["q_bits"][0], "f32") * np.float32(3.0), "f32")
    out = h.gpu.compute_attention(0, h.to_dev(q3))
    bits = out.view(torch.int32).cpu().numpy().view(np.uint32)
    st3 = check_close(bits, h.ora.attend(res["ora_plan"], 0, q3), dtype="f32")
    log(f"f32 D=64 sharpened: {st3}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_f32_d128_scale_phase_and_rope():
    """D=128 (2 heads, 30 frames); a first step of S frames at D=64; and the
    rotary entry points on float32 (K turned in the append, q in one pass):
    pools bit-exact with the oracle's rope_fp64, outputs within the float32
    bounds."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(30,), head_dim=128, dtype="f32")
    h = Harness(wl)
    for t in range(max(wl.frames)):
        res = h.step(run=t in (1, 29), check=t in (1, 29))
        if t in (1, 29):
            st = check_close(res["out_bits"][0], res["ref"][0], dtype="f32")
            log(f"f32 D=128 step {t}: {st}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(12,), dtype="f32")
    S = wl.scale_frames
    h = Harness(wl, max_frames_per_step=S, rope=True)
    res = h.step(check=True, nframes={0: S})
    st = check_close(res["out_bits"][0], res["ref"][0], dtype="f32")
    log(f"f32 scale step with rope: {st}")
    for t in range(1, max(wl.frames) - S + 1):
        res = h.step(check=True)
        check_close(res["out_bits"][0], res["ref"][0], dtype="f32")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)
