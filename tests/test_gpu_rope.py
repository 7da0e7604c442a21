"""Rotary position embedding on the HIP path ([p2] "How LingBot-Map Uses
FlashInfer KV Cache for Streaming 3D Reconstruction" §3D RoPE Position
Encoding): K is turned inside the append kernel on its way into the pool
(kvc_append_frames_rope), q by one pass before attention (kvc_run_rope),
both with caller float32 cos/sin tables, computed in float64 and rounded once
to the element type.  The oracle's rope_fp64 does the same arithmetic, so the
pools must match it bit for bit, a run on device-rotated queries must equal
bitwise a plain run on the oracle's rotated queries, and the outputs must be
within the attention tolerance of the oracle on the rotated rows."""
import dataclasses

import numpy as np
import pytest

import kvc_synth as syn
from oracle import kvc_oracle as ko
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


def test_rope_tiny_every_step_pools_bitexact():
    """The tiny stream (D=32, two blocks) at every step, bf16 and f16."""
    _need_gpu()
    for dtype in ("bf16", "f16"):
        wl = dataclasses.replace(syn.WORKLOADS["tiny"], dtype=dtype)
        h = Harness(wl, num_blocks=2, oracle_blocks=(0, 1), rope=True)
        for t in range(max(wl.frames)):
            res = h.step(check=True)
            _plans_equal(res)
            for b in (0, 1):
                st = check_close(res["out_bits"][b], res["ref"][b], dtype=dtype)
                assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data), f"{dtype} pool block {b} step {t}"
        log(f"rope tiny {dtype} ok {st}")


def test_rope_query_pass_bitexact_and_identity_tables():
    """At D=64 over 70 frames (several splits): kvc_run_rope equals bitwise
    kvc_run on the oracle's rope_fp64 of the same queries; with identity
    tables (cos 1, sin 0) it equals kvc_run on the raw queries; the pool
    holds the oracle's rotated keys bit for bit."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(70,))
    h = Harness(wl, rope=True)
    last = max(wl.frames) - 1
    for t in range(max(wl.frames)):
        res = h.step(run=t in (0, last), check=t in (0, last))
        if t in (0, last):
            _plans_equal(res)
            st = check_close(res["out_bits"][0], res["ref"][0])
            log(f"rope D=64 step {t}: splits {res['gpu_plan']['n_splits']} {st}")
    q_raw, q_rot = res["q_raw"][0], res["q_bits"][0]
    plain = h.gpu.compute_attention(0, h.to_dev(q_rot))
    plain_bits = plain.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(plain_bits, res["out_bits"][0])
    R, half = q_raw.shape[0], wl.head_dim // 2
    one = torch.ones((R, half), dtype=torch.float32, device=h.device)
    zero = torch.zeros_like(one)
    ident = h.gpu.compute_attention(0, h.to_dev(q_raw), rope=(one, zero))
    raw = h.gpu.compute_attention(0, h.to_dev(q_raw))
    assert torch.equal(ident.view(torch.int16), raw.view(torch.int16))
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_rope_f16_d128_and_scale_phase():
    """D=128 with f16 pools over 40 frames, and a first step of S frames
    appended and queried together (the tables of S frames at once)."""
    _need_gpu()
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=2, frames=(40,), head_dim=128, dtype="f16")
    h = Harness(wl, rope=True)
    for t in range(max(wl.frames)):
        res = h.step(run=t in (2, 39), check=t in (2, 39))
        if t in (2, 39):
            _plans_equal(res)
            st = check_close(res["out_bits"][0], res["ref"][0], dtype="f16")
            log(f"rope f16 D=128 step {t}: {st}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)
    wl = dataclasses.replace(syn.WORKLOADS["base"], num_heads=4, frames=(20,))
    S = wl.scale_frames
    h = Harness(wl, num_blocks=2, max_frames_per_step=S, oracle_blocks=(0, 1), rope=True)
    res = h.step(check=True, nframes={0: S})
    for b in (0, 1):
        st = check_close(res["out_bits"][b], res["ref"][b])
        assert np.array_equal(h.pool_bits(b), h.ora.pools[b].data)
    log(f"rope scale-phase step: {st}")
    for t in range(1, max(wl.frames) - S + 1):
        res = h.step(run=t == max(wl.frames) - S, check=t == max(wl.frames) - S)
    check_close(res["out_bits"][0], res["ref"][0])
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_rope_base_full_size():
    """The 256-patch, 64-frame-window workload at H=16, D=64 over its 200
    frames with rotated q and k: outputs at ragged and steady-state steps
    within tolerance, the pool bit-exact at the end."""
    _need_gpu()
    wl = syn.WORKLOADS["base"]
    checks = {0, 72, 199}
    h = Harness(wl, rope=True)
    for t in range(max(wl.frames)):
        res = h.step(run=t in checks, check=t in checks)
        if t in checks:
            _plans_equal(res)
            st = check_close(res["out_bits"][0], res["ref"][0])
            log(f"rope base step {t}: splits {res['gpu_plan']['n_splits']} {st}")
    assert np.array_equal(h.pool_bits(0), h.ora.pools[0].data)


def test_rope_argument_errors():
    """Tables of the wrong shape, type or alignment are refused before any
    launch; no_alloc has no rotary variant."""
    _need_gpu()
    import paged_kv_cache_kvc_amd as kvc
    wl = syn.WORKLOADS["tiny"]
    h = Harness(wl)
    T, H, D = wl.tokens_per_frame, wl.num_heads, wl.head_dim
    k = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    good = torch.zeros((T, D // 2), dtype=torch.float32, device="cuda")
    for bad in (torch.zeros((T, D), dtype=torch.float32, device="cuda"),
                torch.zeros((T, D // 2), dtype=torch.float64, device="cuda"),
                torch.zeros((T * D // 2 + 1,), dtype=torch.float32, device="cuda")[1:].view(T, D // 2)):
        with pytest.raises(kvc.KvcError) as e:
            h.gpu.append_frame(0, k, k, rope=(good, bad))
        assert e.value.status == kvc.KVC_ERR_ARG
    h.gpu.append_frame(0, k, k, rope=(good, good))
    h.gpu.evict_frames(0)
    h.gpu.plan()
    q = torch.zeros_like(k)
    out = torch.empty_like(k)
    with pytest.raises(kvc.KvcError):
        h.gpu.compute_attention(0, q, out=out, no_alloc=True, rope=(good, good))
    lib = kvc.load_library()
    rc = lib.kvc_run_rope(h.gpu._ctx, 0, q.data_ptr(), good.data_ptr() + 4, good.data_ptr(), out.data_ptr(), None)
    assert rc == kvc.KVC_ERR_ARG
    h.gpu.compute_attention(0, q, out=out, rope=(good, good))
    torch.cuda.synchronize()
