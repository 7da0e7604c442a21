#!/usr/bin/env python3
"""Throughput of the two-stream paged KV-cache attention hot path on one GPU.

A step is one frame step of the whole path: for every stream, the new frame
is appended to every block's pool, the window is evicted, one plan is built
and uploaded, and paged attention runs for every block.  The default
workload is the 256-patch, 64-frame-window stream (24 blocks, H=16, D=64,
256 patch + 6 special tokens per frame, page_size 256, 8 scale frames, 200
frames); the timed steps are the last --steps frames of the 200-frame stream,
preceded by --warmup full steps and an untimed append-only fast-forward.

Inputs are synthetic: a device-resident bank of distinct seeded N(0,1) bf16
frames per block, indexed by frame.  Everything timed is resident in HBM
when timing starts.

Two timed regions: the --steps whole steps, with no per-launch events (an
event recorded between two kernels leaves the GPU idle for several
microseconds, which a caller would not pay), give frame-steps/s; then the
attention launches of the last step's blocks, repeated --steps times with
HIP events around each launch on the launch stream, give the kernel's
average duration for the roofline.

Prints one JSON line: frame-steps/s, the roofline of a block's attention
(algorithmic bytes or FLOP per block over the HIP-event-measured duration of
the attention and merge kernels; the attention kernel alone and the whole
step are reported beside it), and the CPU oracle timed on the host as a
reported baseline.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "frame-steps/sec (all blocks) + attn TFLOP/s & HBM GB/s vs MI355X peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 / fp16 MFMA
PEAK_F32_TFLOPS = 157.3     # dense fp32 MFMA


def elem_bytes(dtype):
    return 4 if dtype == "f32" else 2


def mfma_peak(dtype):
    """Dense MFMA peak (TFLOP/s) of the type the attention computes in."""
    return PEAK_F32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
BANK = 8


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KERNEL_SOURCES = ("kvc_kernels.hip", "kvc_attn.hip", "kvc_device.h", "kvc_kernels.h", "kvc_plan_layout.h")


def kernel_source_hash():
    """First 16 hex digits of the SHA-256 of the device code's sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_kvc_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attention_kernel_name(cache, dtype="bf16"):
    """The attention kernel of the cache's current plan: the float32 kernel
    for float32 pools; for the 16-bit types the 32x32 kernel (groups of 256
    or 272 query rows: head_dim 32, and 64 unless the planner took the other)
    or the 16x16 one (groups of 128 or 144 rows: head_dim 128, and 64 where
    fewer query tiles would leave compute units idle)."""
    if dtype == "f32":
        return "attn_f32_kernel"
    return "attn32_kernel" if cache.get_plan_shape()["group_rows"] >= 256 else "attn_kernel"


def read_traffic(workload, kernel):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, calibrated against a plain copy), or
    None when it is missing or was taken on other kernel source."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(p):
        return None
    fields = {}
    with open(p) as fh:
        for line in fh:
            m = re.match(r"^(hbm_bytes_per_launch|kernel_source_sha256_16):\s*(\S+)\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = fields.get("hbm_bytes_per_launch")
    return float(v) if v is not None else None


def cpu_baseline(wl, seconds):
    """The CPU oracle as it stands, timed on this host: dense float64
    attention (gather of the visible tokens + softmax(QK^T/sqrt(D))V) for the
    blocks of steady-state steps at the end of the stream."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import kvc_synth as syn
    from oracle import kvc_oracle as ko

    T, H, D = wl.tokens_per_frame, wl.num_heads, wl.head_dim
    F = max(wl.frames)
    t = F - 1
    ocfg = ko.OracleConfig(num_heads=H, head_dim=D, tokens_per_frame=T, num_special_tokens=wl.num_special_tokens,
                           page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                           max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages,
                           dtype=wl.dtype)
    vis = set(ko.visible_frames(t, wl.scale_frames, wl.sliding_window))
    cache = {}

    def frame_kv(f):
        if f not in cache:
            args = (T, H, D, wl.num_special_tokens, wl.row_offset)
            real = f in vis
            cache[f] = (syn.frame_tensor(wl.seed, 0, f, 0, "k", *args, patch_real=real, dtype=wl.dtype),
                        syn.frame_tensor(wl.seed, 0, f, 0, "v", *args, patch_real=real, dtype=wl.dtype))
        return cache[f]

    q = syn.frame_tensor(wl.seed, 0, t, 0, "q", T, H, D, wl.num_special_tokens, wl.row_offset, dtype=wl.dtype)
    for f in range(F):
        frame_kv(f)
    blocks = 0
    t0 = time.perf_counter()
    while True:
        k, v = ko.gather_dense(ocfg, t, frame_kv)
        ko.attention_fp64(q, k, v, wl.dtype)
        blocks += 1
        el = time.perf_counter() - t0
        if el >= seconds and blocks >= 1:
            break
    L = k.shape[0]
    threads = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    steps = blocks / wl.num_blocks
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": steps / el,
        "unit": "frame-steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{blocks} block(s) of dense float64 oracle attention (gather + softmax) at frame {F}, "
                   f"T={T}, L={L}, H={H}, D={D}; {el:.1f} s on {threads} BLAS thread(s) of "
                   f"{len(os.sched_getaffinity(0))} available ({cpu_model}); one block's seeded history reused per block; "
                   f"frame-steps/s = blocks/{wl.num_blocks}/s"),
        "gflops": 4.0 * T * L * H * D * blocks / el / 1e9,
    }


def achievable_peaks(torch, dev):
    """Measured ceilings on this GPU, reported beside the spec-sheet peaks:
    a 1 GiB device-to-device copy (bytes read + written per second) and a
    large square bf16 matmul (torch, i.e. hipBLASLt)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    b = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tfs = 2.0 * m ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": copy_gbs, "bf16_gemm_TFLOPs": gemm_tfs,
            "how": "1 GiB device copy x10 (read + write bytes); 8192^3 bf16 torch.matmul x20; HIP events"}


def scale_phase(args, torch, syn, kvc, dev):
    """The scale phase of the base shape: S = 8 frames appended in one step
    to all 24 blocks, then paged attention of their 8 x 262 queries over
    their 8 x 262 tokens for every block ([p2] "How LingBot-Map Uses
    FlashInfer KV Cache for Streaming 3D Reconstruction" §Frame Processing
    Loop).  Each timed step resets the host metadata first (the pools keep
    their contents; only valid slots are read)."""
    wl = syn.WORKLOADS["base"]
    nb, T, H, D, S = wl.num_blocks, wl.tokens_per_frame, wl.num_heads, wl.head_dim, wl.scale_frames
    K, W = args.steps, args.warmup
    cfg = kvc.make_config(nb, H, D, T, wl.num_special_tokens, page_size=wl.page_size, scale_frames=S,
                          sliding_window=wl.sliding_window, max_patch_pages=wl.max_patch_pages,
                          max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset,
                          max_frames_per_step=S, dtype=args.dtype)
    cache = kvc.PagedKVCache(cfg, device=dev)
    if args.query_tile:
        cache.set_option(kvc.KVC_OPT_QUERY_TILE, args.query_tile)
    el = cache.elem_dtype
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    mk = lambda: torch.randn((nb, S * T, H, D), generator=g, device=dev).to(el)
    qb, kb, vb = mk(), mk(), mk()
    ob = torch.empty((S * T, H, D), dtype=el, device=dev)
    hs = torch.cuda.current_stream(dev).cuda_stream

    def step(run_profiled=False):
        cache.reset()
        for b in range(nb):
            cache.raw_append_frames(b, kb[b].data_ptr(), vb[b].data_ptr(), S, 0, hs)
            if b == 0:
                cache.evict_frames(0)
                cache.raw_plan(hs)
            cache.raw_run(b, qb[b].data_ptr(), ob.data_ptr(), hs)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    progress(f"timing {K} scale-phase steps")
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = K / wall
    st = cache.get_cache_stats(0)
    L = (st["scale_pages"] + st["live_pages"]) * wl.patch_tokens + st["special_tokens"]
    eb = elem_bytes(args.dtype)
    peak_mfma = mfma_peak(args.dtype)
    flop = 4.0 * S * T * L * H * D
    byts = 2.0 * eb * L * H * D + 2.0 * eb * S * T * H * D
    # the kernels' durations from per-launch HIP events, attention launches repeated on the last plan
    cache.set_option(kvc.KVC_OPT_PROFILE, 1)
    for k in (kvc.KVC_KERNEL_ATTENTION, kvc.KVC_KERNEL_MERGE):
        cache.profile_read(k, reset=True)
    for _ in range(K):
        for b in range(nb):
            cache.raw_run(b, qb[b].data_ptr(), ob.data_ptr(), hs)
    torch.cuda.synchronize()
    cache.set_option(kvc.KVC_OPT_PROFILE, 0)
    a_ms, a_n = cache.profile_read(kvc.KVC_KERNEL_ATTENTION)
    m_ms, m_n = cache.profile_read(kvc.KVC_KERNEL_MERGE)
    # attention + merge time per block, as for the streaming workloads
    a_s = (a_ms + m_ms) / 1e3 / max(a_n, 1)
    tfl = flop / a_s / 1e12
    gbs = byts / a_s / 1e9
    bound = "hbm" if flop / byts < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"
    roof = ({"bound": "mfma", "achieved": tfl, "peak": peak_mfma, "unit": "TFLOP/s",
             "frac": tfl / peak_mfma, "traffic": None} if bound == "mfma" else
            {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
             "traffic": None})
    peaks = achievable_peaks(torch, dev)
    out = {
        "metric": "scale-phase steps/sec (8 frames appended and attended in one step, all 24 blocks)",
        "value": value, "unit": "scale-phase steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": 1e3 * wall / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": (f"scale: {nb} blocks, H={H}, D={D}, {S} frames of {wl.patch_tokens} patch + "
                                f"{wl.num_special_tokens} special tokens in one step, page_size {wl.page_size}"),
                   "num_blocks": nb, "query_rows": S * T, "visible_tokens": L, "num_heads": H, "head_dim": D},
        "roofline": roof,
        "attention": {"kernel": attention_kernel_name(cache, args.dtype), "launches": a_n, "avg_us": 1e3 * a_ms / max(a_n, 1),
                      "attention_plus_merge_us": 1e6 * a_s, "tflops": tfl, "gbs": gbs,
                      "alg_flop_per_launch": flop, "alg_bytes_per_launch": byts,
                      "merge_avg_us": 1e3 * m_ms / max(m_n, 1), "merge_launches": m_n,
                      "frac_hbm_achievable": gbs / peaks["hbm_copy_GBs"],
                      "frac_mfma_achievable": tfl / peaks["bf16_gemm_TFLOPs"], "achievable_peaks": peaks},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="base", choices=["base", "r518", "long", "frag", "scale"],
                    help="scale: the base shape's scale phase, its 8 first frames appended and attended in one step")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16", "f32"],
                    help="element type of the pools and of q, k, v, o")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--target-wgs", type=int, default=None)
    ap.add_argument("--max-splits", type=int, default=None)
    ap.add_argument("--append", default="fused", choices=["fused", "separate"],
                    help="timed steps: kvc_run_append per block (appends ride on the attention and merge "
                         "launches) or kvc_append_frame + kvc_run")
    ap.add_argument("--query-tile", type=int, default=0, choices=[0, 16, 32],
                    help="head_dim 64: query rows per MFMA tile (0: the planner's choice)")
    ap.add_argument("--no-profile", action="store_true", help="time without per-launch HIP events")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import kvc_synth as syn
    import paged_kv_cache_kvc_amd as kvc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.workload == "scale":
        scale_phase(args, torch, syn, kvc, dev)
        return
    wl = syn.WORKLOADS[args.workload]
    F = max(wl.frames)
    K, W = args.steps, args.warmup
    eb = elem_bytes(args.dtype)
    peak_mfma = mfma_peak(args.dtype)
    if K < 1 or W < 0 or K + W > F:
        print(f"need 1 <= steps and steps + warmup <= {F}", file=sys.stderr)
        sys.exit(2)
    nb, T, H, D = wl.num_blocks, wl.tokens_per_frame, wl.num_heads, wl.head_dim
    ns = wl.num_streams

    cfg = kvc.make_config(nb, H, D, T, wl.num_special_tokens, page_size=wl.page_size, scale_frames=wl.scale_frames,
                          sliding_window=wl.sliding_window, num_streams=ns, max_patch_pages=wl.max_patch_pages,
                          max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset,
                          dtype=args.dtype)
    po = so = None
    if wl.shuffle_free_lists:
        po = syn.free_list_order(wl.seed, wl.max_patch_pages, 0, 0)
        so = syn.free_list_order(wl.seed, wl.max_special_pages, wl.max_patch_pages, 1)
    cache = kvc.PagedKVCache(cfg, device=dev, free_patch_order=po, free_special_order=so)
    if args.target_wgs:
        cache.set_option(kvc.KVC_OPT_TARGET_WORKGROUPS, args.target_wgs)
    if args.max_splits:
        cache.set_option(kvc.KVC_OPT_MAX_SPLITS, args.max_splits)
    if args.query_tile:
        cache.set_option(kvc.KVC_OPT_QUERY_TILE, args.query_tile)

    # device-resident input bank: [stream][bank][block] frames
    progress(f"workload {wl.name}: generating input bank")
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)

    def bank(scale=1.0):
        x = torch.randn((ns, BANK, nb, T, H, D), generator=g, device=dev, dtype=torch.float32)
        return x.mul_(scale).to(cache.elem_dtype)
    qb, kb, vb = bank(), bank(), bank()
    ob = torch.empty((ns * T, H, D), dtype=cache.elem_dtype, device=dev)
    qcat = torch.empty((BANK, nb, ns * T, H, D), dtype=cache.elem_dtype, device=dev)
    for s in range(ns):
        qcat[:, :, s * T:(s + 1) * T] = qb[s]

    hs_obj = torch.cuda.current_stream(dev)
    hs = hs_obj.cuda_stream
    if args.append == "fused":
        cache.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
    frame_of = [0] * ns
    gstep = [0]

    def active():
        return [s for s in range(ns) if gstep[0] >= syn.stream_join_step(wl, s)]

    def kv_ptrs(s, b):
        f = frame_of[s] % BANK
        return kb[s, f, b].data_ptr(), vb[s, f, b].data_ptr()

    def step(run):
        act = active()
        fuse = run and args.append == "fused"
        for s in act:
            if fuse:
                cache.append_frames(0, num_frames=1, stream_id=s, stream=hs_obj, defer=True)
            else:
                kp, vp = kv_ptrs(s, 0)
                cache.raw_append(0, kp, vp, s, hs)
        for s in act:
            cache.evict_frames(s)
        cache.raw_plan(hs)          # a plan closes every step, timed or not
        if run:
            if len(act) != ns:
                raise RuntimeError("timed steps must advance every stream")
            qf = qcat[frame_of[0] % BANK]
        for b in range(nb):
            if fuse:
                # the appends of this block ride on its attention and merge launches
                ptrs = [kv_ptrs(s, b) for s in range(ns)]
                cache.raw_run_append(b, [x[0] for x in ptrs], [x[1] for x in ptrs], qf[b].data_ptr(),
                                     ob.data_ptr(), hs)
                continue
            if b > 0:
                for s in act:
                    kp, vp = kv_ptrs(s, b)
                    cache.raw_append(b, kp, vp, s, hs)
            if run:
                cache.raw_run(b, qf[b].data_ptr(), ob.data_ptr(), hs)
        for s in act:
            frame_of[s] += 1
        gstep[0] += 1

    total_steps = F
    ff = total_steps - K - W
    progress(f"fast-forward {ff} append-only steps")
    for i in range(ff):
        step(False)
        if i % 1000 == 999:
            torch.cuda.synchronize()
            progress(f"  {i + 1} steps")
    for _ in range(W):
        step(True)
    torch.cuda.synchronize()

    # algorithmic work per timed step: visible valid tokens from the cache stats
    def step_work():
        fl = by = 0.0
        for s in range(ns):
            st = cache.get_cache_stats(s)
            L = (st["scale_pages"] + st["live_pages"]) * wl.patch_tokens + st["special_tokens"]
            fl += 4.0 * T * L * H * D
            by += 2.0 * eb * L * H * D + 2.0 * eb * T * H * D   # K and V read once, Q read, O written
        return fl, by

    # Timed region 1: K whole steps with no per-launch events (the events
    # themselves would insert an idle gap at every kernel boundary).
    progress(f"timing {K} steps")
    flops = bytes_ = 0.0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        step(True)
        fl, by = step_work()
        flops += fl * nb
        bytes_ += by * nb
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    elapsed = max(wall, gpu_ms / 1e3)
    value = K / elapsed
    out = {
        "metric": METRIC, "value": value, "unit": "frame-steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": 1e3 * elapsed / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": (f"{wl.name}: {nb} blocks, H={H}, D={D}, {wl.patch_tokens} patch + "
                                f"{wl.num_special_tokens} special tokens/frame, page_size {wl.page_size}, "
                                f"scale {wl.scale_frames}, window {wl.sliding_window}, streams {ns} at "
                                f"{list(wl.frames)} frames; timed steps = last {K} frames"),
                   "num_blocks": nb, "tokens_per_frame": T, "num_heads": H, "head_dim": D,
                   "page_size": wl.page_size, "frames": list(wl.frames), "streams": ns},
    }
    if not args.no_profile:
        # Timed region 2: the kernels' durations, from HIP events that the
        # library records around each of its launches on the launch stream.
        # The attention (and merge) launches of the last step's 24 blocks are
        # repeated K times on that step's plan: the same work as a timed step.
        cache.set_option(kvc.KVC_OPT_PROFILE, 1)
        for k in (kvc.KVC_KERNEL_ATTENTION, kvc.KVC_KERNEL_MERGE):
            cache.profile_read(k, reset=True)
        progress(f"timing the attention launches of {K} steps with per-launch HIP events")
        fl, by = step_work()
        pf, pb = fl * nb * K, by * nb * K
        qf = qcat[(frame_of[0] - 1) % BANK]
        for _ in range(K):
            for b in range(nb):
                cache.raw_run(b, qf[b].data_ptr(), ob.data_ptr(), hs)
        torch.cuda.synchronize()
        cache.set_option(kvc.KVC_OPT_PROFILE, 0)
        a_ms, a_n = cache.profile_read(kvc.KVC_KERNEL_ATTENTION)
        m_ms, m_n = cache.profile_read(kvc.KVC_KERNEL_MERGE)
        # Throughput over attention + merge time (the split-KV merge is part
        # of the attention of a block); the attention kernel alone and the
        # whole step (append, plan and launches included) are reported too.
        am_s = (a_ms + m_ms) / 1e3
        gbs = pb / am_s / 1e9
        tfl = pf / am_s / 1e12
        gbs_a = pb / (a_ms / 1e3) / 1e9
        tfl_a = pf / (a_ms / 1e3) / 1e12
        step_s = elapsed / K
        gbs_step = pb / K / step_s / 1e9
        tfl_step = pf / K / step_s / 1e12
        bound = "hbm" if pf / pb < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"
        kname = attention_kernel_name(cache, args.dtype)
        traffic = read_traffic(wl.name, kname)
        if bound == "hbm":
            roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                    "frac_attention_kernel_only": gbs_a / PEAK_HBM_GBS, "frac_whole_step": gbs_step / PEAK_HBM_GBS}
        else:
            roof = {"bound": "mfma", "achieved": tfl, "peak": peak_mfma, "unit": "TFLOP/s",
                    "frac": tfl / peak_mfma, "frac_attention_kernel_only": tfl_a / peak_mfma,
                    "frac_whole_step": tfl_step / peak_mfma}
        roof["traffic"] = traffic
        roof["time"] = "attention + merge kernels, per block (HIP events)"
        out["roofline"] = roof
        peaks = achievable_peaks(torch, dev)
        out["attention"] = {
            "kernel": kname, "launches": a_n, "avg_us": 1e3 * a_ms / max(a_n, 1),
            "tflops": tfl_a, "gbs": gbs_a, "frac_hbm": gbs_a / PEAK_HBM_GBS, "frac_mfma": tfl_a / peak_mfma,
            "alg_bytes_per_launch": pb / max(a_n, 1), "alg_flop_per_launch": pf / max(a_n, 1),
            "merge_avg_us": 1e3 * m_ms / max(m_n, 1), "merge_launches": m_n,
            "attention_plus_merge_us": 1e6 * am_s / max(a_n, 1),
            "frac_hbm_achievable": gbs / peaks["hbm_copy_GBs"],
            "frac_mfma_achievable": tfl / peaks["bf16_gemm_TFLOPs"],
            "achievable_peaks": peaks,
            "timing": ("per-launch HIP events on the launch stream, around the attention and merge launches of "
                       "the last timed step repeated K times (value is timed without per-launch events)"),
        }
    progress(json.dumps({k: out[k] for k in ("value", "ms_per_step")}))
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle")
        import dataclasses
        out["cpu_baseline"] = cpu_baseline(dataclasses.replace(wl, dtype=args.dtype), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
