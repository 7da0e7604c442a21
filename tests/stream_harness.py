"""Drives the HIP library and the CPU oracle through the same synthetic frame
stream (test helper; used by the GPU parity tests, the smoke check and the
bench's parity spot check)."""
from __future__ import annotations

import time
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

import kvc_synth as syn
from oracle import kvc_oracle as ko


def cfg_args(wl: syn.Workload, num_blocks: int):
    return dict(num_blocks=num_blocks, num_heads=wl.num_heads, head_dim=wl.head_dim,
                tokens_per_frame=wl.tokens_per_frame, num_special_tokens=wl.num_special_tokens,
                page_size=wl.page_size, scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                num_streams=wl.num_streams, max_patch_pages=wl.max_patch_pages,
                max_special_pages=wl.max_special_pages, special_row_offset=wl.row_offset, dtype=wl.dtype)


def oracle_cfg(wl: syn.Workload) -> ko.OracleConfig:
    return ko.OracleConfig(num_heads=wl.num_heads, head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame,
                           num_special_tokens=wl.num_special_tokens, page_size=wl.page_size,
                           scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                           max_patch_pages=wl.max_patch_pages, max_special_pages=wl.max_special_pages,
                           num_streams=wl.num_streams, special_row_offset=wl.special_row_offset,
                           dtype=wl.dtype)


def edge_workloads() -> Dict[str, syn.Workload]:
    """Degenerate shapes: frames without special tokens, the most special
    tokens a frame may carry (64, spanning four 16-slot pages), one-token
    frames on a single head at D=128, and the most frames one step may append
    (64, a scale phase of 64 tiny frames followed by single frames)."""
    W = syn.Workload
    return {
        "no_specials": W("no_specials", 1, 2, 64, 20, 0, 20, 2, 3, (10,), 21,
                         max_patch_pages=2 + 3 + 1, max_special_pages=0),
        "max_specials": W("max_specials", 1, 2, 32, 16, 64, 16, 1, 2, (6,), 22,
                          max_patch_pages=1 + 2 + 1, max_special_pages=24),
        "one_token": W("one_token", 1, 1, 128, 1, 0, 1, 1, 3, (8,), 23,
                       max_patch_pages=1 + 3 + 1, max_special_pages=0),
        "steps_of_64": W("steps_of_64", 1, 2, 32, 16, 6, 16, 8, 64, (74,), 24,
                         max_patch_pages=8 + 64 + 1, max_special_pages=28),
    }


def free_orders(wl: syn.Workload, seed: Optional[int] = None):
    if seed is None:
        if not wl.shuffle_free_lists:
            return None, None
        seed = wl.seed
    return (syn.free_list_order(seed, wl.max_patch_pages, 0, 0),
            syn.free_list_order(seed, wl.max_special_pages, wl.max_patch_pages, 1))


def final_visible(wl: syn.Workload, stream: int, extra_steps: Sequence[int] = ()) -> set:
    """Frames of a stream whose patch rows are visible at its last step or at
    any of the given (stream-local) steps."""
    F = wl.frames[stream]
    out = set()
    for t in [F - 1, *extra_steps]:
        out.update(ko.visible_frames(t, wl.scale_frames, wl.sliding_window))
    return out


def bits_to_f32(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    return syn.bits_to_f32(bits, dtype)


# Error model of the kernels' output, relative to the float64 oracle, for
# 16-bit inputs (bf16 has 8 significant bits, f16 11):
#   * the probabilities are rounded toward zero to the element type before
#     the P.V product (relative error below 2^-7 for bf16), and the row sums
#     are taken over the same rounded values, so only the spread of that
#     error around its mean reaches the output: about 2^-7/sqrt(12) times the
#     weighted spread of the values, small unless one key dominates;
#   * each split's normalised partial output is rounded to the element type
#     (relative 2^-9), and the merged output once more (2^-9).
# Both rounding terms scale with the output's own magnitude, so the error's
# RMS over a launch is of order 2^-9 of the output's RMS, and its largest
# value a few 2^-9 of the largest partial.  The bounds below leave a margin of
# about 4x over that model while failing any kernel whose error is a visible
# fraction of the output's spread (the absolute tolerance alone would not at
# long contexts, where the output's std falls to about 0.01).
REL_RMS_BOUND = 2.0 ** -6       # ||o - o_ref|| / ||o_ref||, bf16
MAX_OVER_STD_BOUND = 0.25       # max |o - o_ref| / std(o_ref), bf16
# f16 keeps 3 more significant bits: every term above shrinks by 8
BOUNDS = {"bf16": (REL_RMS_BOUND, MAX_OVER_STD_BOUND), "f16": (REL_RMS_BOUND / 8, MAX_OVER_STD_BOUND / 8)}
# float32 pools: nothing is rounded to 16 bits; what remains is float32
# arithmetic (products and sums in the MFMA, 2^-24 relative per operation,
# growing with the square root of the terms summed) and the exponential's
# ulp error: about 2^-20 relative to the output, bounded here with a margin
# of 16x.  The elementwise test uses ELEMENT_TOL["f32"].
BOUNDS["f32"] = (2.0 ** -16, 2.0 ** -12)
ELEMENT_TOL = {"bf16": (1e-2, 1e-2), "f16": (1e-2, 1e-2), "f32": (1e-5, 1e-4)}


def np_bits(dtype: str):
    """numpy and torch integer types of the element type's bit patterns."""
    import torch
    return (np.uint32, torch.int32, np.int32) if dtype == "f32" else (np.uint16, torch.int16, np.int16)


def check_close(out_bits: np.ndarray, ref: np.ndarray, atol=None, rtol=None, dtype: str = "bf16",
                rel_rms_bound: Optional[float] = None, max_over_std_bound: Optional[float] = None
                ) -> Dict[str, float]:
    """The acceptance test: |o - o_ref| <= atol + rtol * |o_ref| elementwise
    (the stated tolerance), and the relative RMS error and the largest error
    over the output's standard deviation within the rounding-model bounds
    above; returns error statistics."""
    if atol is None:
        atol = ELEMENT_TOL[dtype][0]
    if rtol is None:
        rtol = ELEMENT_TOL[dtype][1]
    if rel_rms_bound is None:
        rel_rms_bound = BOUNDS[dtype][0]
    if max_over_std_bound is None:
        max_over_std_bound = BOUNDS[dtype][1]
    o = bits_to_f32(out_bits, dtype).astype(np.float64)
    err = np.abs(o - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    std = max(float(ref.std()), 1e-30)
    stats = {"max_abs": float(err.max()), "max_over_std": float(err.max() / std),
             "rel_rms": float(np.sqrt((err ** 2).sum() / max(float((ref ** 2).sum()), 1e-300))),
             "frac_over_half_tol": float((err > 0.5 * bound).mean()), "n_bad": int(bad.sum())}
    assert not bad.any(), f"{bad.sum()} elements out of tolerance; {stats}"
    assert stats["rel_rms"] <= rel_rms_bound, f"relative RMS error above {rel_rms_bound}; {stats}"
    assert stats["max_over_std"] <= max_over_std_bound, f"max error / std above {max_over_std_bound}; {stats}"
    return stats


def check_split_matches_unsplit(a: np.ndarray, b: np.ndarray):
    """Elementwise: a split run and an unsplit run of the same attention
    differ by the rounding of the split partials (2^-9 of a partial, whose
    magnitude can reach a few times the output's spread) and of the
    probabilities.  |a - b| <= 2^-7 |b| + 2^-4 std(b) for every element."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    lim = 2.0 ** -7 * np.abs(b) + 2.0 ** -4 * b.std()
    d = np.abs(a - b)
    assert (d <= lim).all(), f"{int((d > lim).sum())} elements differ beyond the bound; max {d.max()} (std {b.std()})"
    return float(d.max() / b.std())


class Harness:
    """The GPU cache and the oracle side by side.

    blocks: how many block pools to exercise (block b draws its inputs with
    block index b).  real_patch(stream, frame) says whether a frame's patch
    rows are drawn (else zero; only for frames never visible at a checked
    step).  rope: K is appended through kvc_append_frames_rope and q run
    through kvc_run_rope with the tables of kvc_synth.rope_tables for each
    frame; the oracle sees rope_fp64 of the same rows.  fused: plans built
    with KVC_OPT_FUSED_APPEND; every block that runs defers its appends and
    runs through kvc_run_append, the others append with their rows."""

    def __init__(self, wl: syn.Workload, num_blocks: int = 1, q_scale: float = 1.0,
                 real_patch: Optional[Callable[[int, int], bool]] = None, orders=None,
                 options: Optional[Dict[int, int]] = None, device="cuda", oracle_blocks: Sequence[int] = (0,),
                 max_frames_per_step: int = 1, rope: bool = False, fused: bool = False):
        import torch
        import paged_kv_cache_kvc_amd as kvc
        self.torch = torch
        self.kvc = kvc
        self.wl = wl
        self.nb = num_blocks
        self.q_scale = q_scale
        self.real_patch = real_patch or (lambda s, f: True)
        po, so = orders if orders is not None else free_orders(wl)
        self.gpu = kvc.PagedKVCache(kvc.make_config(**cfg_args(wl, num_blocks),
                                                    max_frames_per_step=max_frames_per_step), device=device,
                                    free_patch_order=po, free_special_order=so)
        assert not (fused and rope), "the fused append takes no rotary tables"
        self.fused = fused
        if fused:
            self.gpu.set_option(kvc.KVC_OPT_FUSED_APPEND, 1)
        for k, v in (options or {}).items():
            self.gpu.set_option(k, v)
        self.ocfg = oracle_cfg(wl)
        self.ora = ko.OracleStream(self.ocfg, blocks=tuple(oracle_blocks), free_patch_order=po,
                                   free_special_order=so)
        self.global_step = 0
        self.frame_of = [0] * wl.num_streams
        # frames drawn but rolled back per stream: the oracle numbers frames by
        # its allocator's count, the inputs are drawn by frame_of
        self.skew = [0] * wl.num_streams
        T, H, D = wl.tokens_per_frame, wl.num_heads, wl.head_dim
        self.kbuf = torch.empty((T, H, D), dtype=self.gpu.elem_dtype, device=device)
        self.vbuf = torch.empty_like(self.kbuf)
        self.device = device
        self.rope = rope

    def tables(self, f: int, n: int = 1):
        """Rotary tables (float32 cos, sin [n * T, D/2]) of drawn frames f ..
        f + n - 1."""
        wl = self.wl
        return syn.rope_tables(f, n, wl.tokens_per_frame, wl.head_dim, wl.num_special_tokens, wl.row_offset)

    def tables_dev(self, tabs):
        return tuple(self.torch.from_numpy(t).to(self.device) for t in tabs)

    def _frame(self, s, f, b, which):
        wl = self.wl
        return syn.frame_tensor(wl.seed, s, f, b, which, wl.tokens_per_frame, wl.num_heads, wl.head_dim,
                                wl.num_special_tokens, wl.row_offset,
                                scale=self.q_scale if which == "q" else 1.0,
                                patch_real=self.real_patch(s, f) or which == "q", dtype=wl.dtype)

    def to_dev(self, bits: np.ndarray, out=None):
        t = self.torch.from_numpy(np.ascontiguousarray(bits).view(np_bits(self.wl.dtype)[2])).view(self.gpu.elem_dtype)
        if out is None:
            return t.to(self.device)
        out.copy_(t)
        return out

    def active(self) -> List[int]:
        return [s for s in range(self.wl.num_streams) if self.global_step >= syn.stream_join_step(self.wl, s)]

    def step(self, run: bool = True, check: bool = False, blocks_to_run: Optional[Sequence[int]] = None,
             nframes: Optional[Dict[int, int]] = None):
        """One step for every active stream: one frame each, or nframes[s]
        frames (a scale-phase step).  Returns a dict with the GPU outputs
        (bits per block) and, when check, the oracle outputs and plans."""
        act = self.active()
        frames = {s: self.frame_of[s] for s in act}
        nf = {s: (nframes or {}).get(s, 1) for s in act}
        kv_cache = {}

        def frame_kv(s, f, b):
            key = (s, f, b)
            if key not in kv_cache:
                kv_cache[key] = (self._frame(s, f, b, "k"), self._frame(s, f, b, "v"))
            return kv_cache[key]

        def frame_kv_oracle(s, f, b):
            k, v = frame_kv(s, f, b)
            if self.rope:
                k = ko.rope_fp64(k, *self.tables(f), self.wl.dtype)
            return k, v

        res = {"active": act, "frames": frames}
        run_blocks = list(range(self.nb)) if blocks_to_run is None else list(blocks_to_run)
        outs = {}
        for b in range(self.nb):
            fuse_b = self.fused and run and b in run_blocks
            kin, vin = {}, {}
            for s in act:
                rope = self.tables_dev(self.tables(frames[s], nf[s])) if self.rope else None
                if fuse_b:
                    kvs = [frame_kv(s, frames[s] + j, b) for j in range(nf[s])]
                    kin[s] = self.to_dev(np.concatenate([x[0] for x in kvs]))
                    vin[s] = self.to_dev(np.concatenate([x[1] for x in kvs]))
                    self.gpu.append_frames(b, num_frames=nf[s], stream_id=s, defer=True)
                elif nf[s] == 1:
                    k, v = frame_kv(s, frames[s], b)
                    self.to_dev(k, self.kbuf)
                    self.to_dev(v, self.vbuf)
                    self.gpu.append_frame(b, self.kbuf, self.vbuf, stream_id=s, rope=rope)
                else:
                    kvs = [frame_kv(s, frames[s] + j, b) for j in range(nf[s])]
                    kd = self.to_dev(np.concatenate([x[0] for x in kvs]))
                    vd = self.to_dev(np.concatenate([x[1] for x in kvs]))
                    self.gpu.append_frames(b, kd, vd, num_frames=nf[s], stream_id=s, rope=rope)
            if b == 0:
                for s in act:
                    self.gpu.evict_frames(s)
                self.gpu.plan()           # a plan closes every step, run or not
            if run and b in run_blocks:
                q = np.concatenate([self._frame(s, frames[s] + j, b, "q") for s in act for j in range(nf[s])])
                qd = self.to_dev(q)
                if self.rope:
                    tabs = [np.concatenate(x) for x in zip(*(self.tables(frames[s], nf[s]) for s in act))]
                    out = self.gpu.compute_attention(b, qd, rope=self.tables_dev(tabs))
                    res.setdefault("q_raw", {})[b] = q
                    q = ko.rope_fp64(q, *tabs, self.wl.dtype)
                elif fuse_b:
                    out = self.gpu.append_run(b, kin, vin, qd)
                else:
                    out = self.gpu.compute_attention(b, qd)
                outs[b] = (q, out)
        # oracle replay (allocator always; pools only for its blocks)
        ora_plan = self.ora.step(act, lambda s, f, b: frame_kv_oracle(s, f + self.skew[s], b),
                                 frames=[nf[s] for s in act])
        res["ora_plan"] = ora_plan
        res["gpu_plan"] = self.gpu.get_plan()
        nb, tb, _ = np_bits(self.wl.dtype)
        res["out_bits"] = {b: out.view(tb).cpu().numpy().view(nb) for b, (q, out) in outs.items()}
        res["q_bits"] = {b: q for b, (q, out) in outs.items()}
        if check:
            res["ref"] = {b: self.ora.attend(ora_plan, b, q) for b, (q, out) in outs.items() if b in self.ora.pools}
        for s in act:
            self.frame_of[s] += nf[s]
        self.global_step += 1
        return res

    def rollback(self, s: int):
        """Undo stream s's most recent frame on both sides.  The next frame
        draws new inputs, so rows left behind by the undone frame would show."""
        self.gpu.rollback_frame(s)
        self.ora.alloc.rollback_frame(s)
        self.skew[s] += 1

    def pool_bits(self, block: int) -> np.ndarray:
        nb, tb, _ = np_bits(self.wl.dtype)
        return self.gpu.pools[block].view(tb).cpu().numpy().view(nb)
