"""Two-stream paged KV-cache prefill attention for MI355X (gfx950).

Thin Python binding over the C-ABI of libkvc.so (include/kvc.h): argument
marshalling only.  Every step of the path (page allocation, planning, append,
attention, merge) runs in the native library; PyTorch provides device memory
and streams.

Method names follow the cache manager described in [p1] "How FlashInfer KV
Cache Attention Accelerates Streaming 3D Reconstruction Over SDPA"
§FlashInferKVCacheManager Responsibilities (append_frame, evict_frames,
compute_attention, reset) and [p3] "How FlashInfer's Paged KV Cache Attention
Outperforms SDPA Fallback in Streaming Inference" §Inspecting Cache Statistics
(get_cache_stats).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK = 0
KVC_ERR_ARG = -1
KVC_ERR_STATE = -2
KVC_ERR_POOL_EXHAUSTED = -3
KVC_ERR_CAPACITY = -4
KVC_ERR_HIP = -5
KVC_ERR_UNSUPPORTED = -6
KVC_ERR_HOST_ALLOC = -7
NO_ALLOC_SCRATCH_BYTES = 64 << 20   # KVC_NO_ALLOC_SCRATCH_BYTES of include/kvc.h

KVC_OPT_TARGET_WORKGROUPS = 1
KVC_OPT_MAX_SPLITS = 2
KVC_OPT_PROFILE = 3
KVC_OPT_DEFER_EVICTION = 4
KVC_OPT_QUERY_TILE = 5
KVC_OPT_FUSED_APPEND = 6
KVC_DTYPE_BF16 = 0
KVC_DTYPE_F16 = 1
KVC_DTYPE_F32 = 2
DTYPES = {"bf16": KVC_DTYPE_BF16, "f16": KVC_DTYPE_F16, "f32": KVC_DTYPE_F32}

KVC_KERNEL_ATTENTION = 0
KVC_KERNEL_MERGE = 1
KVC_KERNEL_APPEND = 2
KVC_KERNEL_ROPE = 3

MAX_SPLITS = 64
ABI_VERSION = 8   # KVC_ABI_VERSION of include/kvc.h


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvc error {status}: {message}")
        self.status = status


class KvcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "num_heads", "head_dim", "tokens_per_frame", "num_special_tokens",
        "special_row_offset", "page_size", "scale_frames", "sliding_window", "num_streams",
        "max_patch_pages", "max_special_pages", "max_frames_per_step", "dtype")]


class KvcStats(ctypes.Structure):
    _fields_ = [("frame_count", ctypes.c_int64), ("special_tokens", ctypes.c_int64),
                ("scale_pages", ctypes.c_int32), ("live_pages", ctypes.c_int32),
                ("free_pages", ctypes.c_int32), ("special_pages", ctypes.c_int32),
                ("free_special_pages", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# every exported symbol of include/kvc.h with (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)
SIGNATURES = {
    "kvc_abi_version": (_I32, []),
    "kvc_status_string": (ctypes.c_char_p, [_I32]),
    "kvc_pool_bytes": (ctypes.c_size_t, [ctypes.POINTER(KvcConfig)]),
    "kvc_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(KvcConfig)]),
    "kvc_staging_bytes": (ctypes.c_size_t, [ctypes.POINTER(KvcConfig)]),
    "kvc_create": (_I32, [ctypes.POINTER(KvcConfig), ctypes.POINTER(_P), _P, _P, _PI32, _PI32, ctypes.POINTER(_P)]),
    "kvc_create_metadata_only": (_I32, [ctypes.POINTER(KvcConfig), _PI32, _PI32, ctypes.POINTER(_P)]),
    "kvc_destroy": (_I32, [_P]),
    "kvc_reset": (_I32, [_P]),
    "kvc_append_frame": (_I32, [_P, _I32, _I32, _P, _P, _P]),
    "kvc_append_frames": (_I32, [_P, _I32, _I32, _P, _P, _I32, _P]),
    "kvc_append_frames_rope": (_I32, [_P, _I32, _I32, _P, _P, _I32, _P, _P, _P]),
    "kvc_evict": (_I32, [_P, _I32]),
    "kvc_rollback": (_I32, [_P, _I32]),
    "kvc_plan": (_I32, [_P, _P]),
    "kvc_run": (_I32, [_P, _I32, _P, _P, _P]),
    "kvc_run_no_alloc": (_I32, [_P, _I32, _P, _P, _P]),
    "kvc_run_append": (_I32, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _P, _P]),
    "kvc_run_rope": (_I32, [_P, _I32, _P, _P, _P, _P, _P]),
    "kvc_get_plan": (_I32, [_P, _PI32, _PI32, _PI32, _PI32, _PI32, _PI32, _PI32, _I32, _I32, _PI32, _PI32]),
    "kvc_get_plan_shape": (_I32, [_P, _PI32, _PI32]),
    "kvc_get_plan_image": (_I32, [_P, _PI32, _I32, _PI32]),
    "kvc_get_split_partials": (_I32, [_P, ctypes.POINTER(ctypes.c_float), ctypes.c_int64,
                                      ctypes.POINTER(ctypes.c_uint16), ctypes.c_int64,
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), _P]),
    "kvc_get_stats": (_I32, [_P, _I32, ctypes.POINTER(KvcStats)]),
    "kvc_set_option": (_I32, [_P, _I32, ctypes.c_int64]),
    "kvc_get_option": (_I32, [_P, _I32, ctypes.POINTER(ctypes.c_int64)]),
    "kvc_profile_read": (_I32, [_P, _I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), _I32]),
    "kvc_last_error": (ctypes.c_char_p, [_P]),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkvc.so; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m paged_kv_cache_kvc_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kvc_abi_version() != ABI_VERSION:
        raise ImportError("libkvc.so ABI version mismatch")
    if path == LIB_PATH:
        _lib = lib
    return lib


def _ceil_div(a, b):
    return -(-a // b)


def make_config(num_blocks, num_heads, head_dim, tokens_per_frame, num_special_tokens=6, page_size=None,
                scale_frames=8, sliding_window=64, num_streams=1, max_patch_pages=None,
                max_special_pages=None, max_total_frames=None, special_row_offset=None,
                max_frames_per_step=1, dtype="bf16") -> KvcConfig:
    """Build a kvc_config.  Defaults follow [p2] §Initializing the Cache
    Manager: page_size = patch tokens, patch pages = S + W + 16 headroom per
    stream, special pages sized for max_total_frames."""
    P = tokens_per_frame - num_special_tokens
    if page_size is None:
        page_size = P
    if max_patch_pages is None:
        max_patch_pages = num_streams * (scale_frames + sliding_window + 16)
    if max_special_pages is None:
        total = 200 if max_total_frames is None else max_total_frames
        max_special_pages = num_streams * _ceil_div(total * num_special_tokens, page_size)
    if special_row_offset is None:
        special_row_offset = P
    if dtype not in DTYPES:
        raise KvcError(KVC_ERR_ARG, f"dtype must be one of {sorted(DTYPES)}")
    return KvcConfig(num_blocks, num_heads, head_dim, tokens_per_frame, num_special_tokens, special_row_offset,
                     page_size, scale_frames, sliding_window, num_streams, max_patch_pages, max_special_pages,
                     max_frames_per_step, DTYPES[dtype])


class PagedKVCache:
    """One cache: per-block page pools, the page lists of each stream and the
    per-step plan.  Device buffers are torch tensors owned here; the library
    only receives their addresses."""

    def __init__(self, config: KvcConfig, device="cuda", free_patch_order: Optional[Sequence[int]] = None,
                 free_special_order: Optional[Sequence[int]] = None, metadata_only: bool = False):
        self.lib = load_library()
        self.cfg = config
        self.metadata_only = metadata_only
        self._ctx = ctypes.c_void_p()
        fpo = self._i32_array(free_patch_order)
        fso = self._i32_array(free_special_order)
        self._planned = False
        self.pools = []
        if metadata_only:
            rc = self.lib.kvc_create_metadata_only(ctypes.byref(config), fpo, fso, ctypes.byref(self._ctx))
            self._check(rc, "kvc_create_metadata_only", ctx=False)
            return
        import torch
        self.torch = torch
        self.elem_dtype = {KVC_DTYPE_BF16: torch.bfloat16, KVC_DTYPE_F16: torch.float16,
                           KVC_DTYPE_F32: torch.float32}[config.dtype]
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        pool_bytes = self.lib.kvc_pool_bytes(ctypes.byref(config))
        ws_bytes = self.lib.kvc_workspace_bytes(ctypes.byref(config))
        st_bytes = self.lib.kvc_staging_bytes(ctypes.byref(config))
        if not pool_bytes or not ws_bytes or not st_bytes:
            raise KvcError(KVC_ERR_ARG, "invalid configuration")
        pages = config.max_patch_pages + config.max_special_pages
        shape = (pages, 2, config.page_size, config.num_heads, config.head_dim)
        with torch.cuda.device(self.device):
            self.pools = [torch.empty(shape, dtype=self.elem_dtype, device=self.device)
                          for _ in range(config.num_blocks)]
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
            self.staging = torch.empty(st_bytes, dtype=torch.uint8, pin_memory=True)
            ptrs = (ctypes.c_void_p * config.num_blocks)(*[p.data_ptr() for p in self.pools])
            rc = self.lib.kvc_create(ctypes.byref(config), ptrs, self.workspace.data_ptr(),
                                     self.staging.data_ptr(), fpo, fso, ctypes.byref(self._ctx))
        self._check(rc, "kvc_create", ctx=False)

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _i32_array(seq):
        if seq is None:
            return None
        arr = np.ascontiguousarray(np.asarray(seq, dtype=np.int32))
        return arr.ctypes.data_as(_PI32)

    def _check(self, rc, what, ctx=True):
        if rc != KVC_OK:
            msg = self.lib.kvc_last_error(self._ctx).decode() if ctx and self._ctx else ""
            name = self.lib.kvc_status_string(rc).decode()
            raise KvcError(rc, f"{what}: {name}{': ' + msg if msg else ''}")

    def _stream(self, stream):
        if stream is None:
            stream = self.torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(stream.cuda_stream)

    def _check_tensor(self, t, rows, name):
        c = self.cfg
        if t.dtype != self.elem_dtype or not t.is_contiguous() or t.device != self.device \
                or tuple(t.shape) != (rows, c.num_heads, c.head_dim):
            raise KvcError(KVC_ERR_ARG, f"{name} must be a contiguous {self.elem_dtype} [{rows}, {c.num_heads}, "
                                        f"{c.head_dim}] tensor on {self.device}")

    def _check_tables(self, rope, rows):
        """Rotary tables (cos, sin): contiguous float32 [rows, D/2] tensors on
        this device, 16-byte aligned."""
        half = self.cfg.head_dim // 2
        if not isinstance(rope, (tuple, list)) or len(rope) != 2:
            raise KvcError(KVC_ERR_ARG, "rope must be a pair (cos, sin)")
        for name, t in zip(("cos", "sin"), rope):
            if t.dtype != self.torch.float32 or not t.is_contiguous() or t.device != self.device \
                    or tuple(t.shape) != (rows, half) or t.data_ptr() % 16:
                raise KvcError(KVC_ERR_ARG, f"rope {name} must be a contiguous 16-byte aligned float32 "
                                            f"[{rows}, {half}] tensor on {self.device}")
        return rope[0].data_ptr(), rope[1].data_ptr()

    # -- the method ------------------------------------------------------
    def append_frame(self, block_idx: int, k=None, v=None, stream_id: int = 0, stream=None, rope=None):
        """Write one frame's K and V ([T, H, D] bf16) of one block; at block 0
        this also allocates the frame's patch page and special slots.  rope =
        (cos, sin), float32 [T, D/2] each, turns K by those angles on the way
        into the pool (kvc_append_frames_rope)."""
        if rope is not None:
            self.append_frames(block_idx, k, v, 1, stream_id, stream, rope)
            return
        if self.metadata_only:
            rc = self.lib.kvc_append_frame(self._ctx, stream_id, block_idx, None, None, None)
        else:
            T = self.cfg.tokens_per_frame
            self._check_tensor(k, T, "k")
            self._check_tensor(v, T, "v")
            rc = self.lib.kvc_append_frame(self._ctx, stream_id, block_idx, k.data_ptr(), v.data_ptr(),
                                           self._stream(stream))
        self._check(rc, "append_frame")
        if block_idx == 0:
            self._planned = False

    def append_frames(self, block_idx: int, k=None, v=None, num_frames: Optional[int] = None, stream_id: int = 0,
                      stream=None, rope=None, defer: bool = False):
        """Write several frames' K and V ([F, T, H, D] or [F*T, H, D] bf16) of
        one block in one step (the scale phase); at block 0 this also
        allocates the F frames, all or none.  rope = (cos, sin), float32
        [F*T, D/2] each, turns K by those angles on the way into the pool.
        defer = True (KVC_OPT_FUSED_APPEND) does the bookkeeping only: the
        block's append_run makes the copy."""
        if defer:
            if num_frames is None or k is not None or v is not None or rope is not None:
                raise KvcError(KVC_ERR_ARG, "a deferred append takes num_frames and no tensors")
            rc = self.lib.kvc_append_frames(self._ctx, stream_id, block_idx, None, None, num_frames,
                                            self._stream(stream))
            self._check(rc, "append_frames")
            if block_idx == 0:
                self._planned = False
            return
        if self.metadata_only:
            if num_frames is None:
                raise KvcError(KVC_ERR_ARG, "num_frames is required without tensors")
            if rope is not None:
                raise KvcError(KVC_ERR_ARG, "a metadata-only cache takes no rotary tables")
            rc = self.lib.kvc_append_frames(self._ctx, stream_id, block_idx, None, None, num_frames, None)
        else:
            T = self.cfg.tokens_per_frame
            F = k.shape[0] if k.dim() == 4 else k.shape[0] // T
            if num_frames is not None and num_frames != F:
                raise KvcError(KVC_ERR_ARG, f"num_frames {num_frames} does not match k ({F} frames)")
            k2 = k.reshape(F * T, *k.shape[-2:])
            v2 = v.reshape(F * T, *v.shape[-2:])
            self._check_tensor(k2, F * T, "k")
            self._check_tensor(v2, F * T, "v")
            if rope is None:
                rc = self.lib.kvc_append_frames(self._ctx, stream_id, block_idx, k2.data_ptr(), v2.data_ptr(), F,
                                                self._stream(stream))
            else:
                cp, sp = self._check_tables(rope, F * T)
                rc = self.lib.kvc_append_frames_rope(self._ctx, stream_id, block_idx, k2.data_ptr(), v2.data_ptr(),
                                                     F, cp, sp, self._stream(stream))
        self._check(rc, "append_frames")
        if block_idx == 0:
            self._planned = False

    def evict_frames(self, stream_id: int = 0, block_idx: Optional[int] = None):
        """Return live-window pages beyond the window to the free list (host
        metadata only, once per step; block_idx is accepted and ignored)."""
        self._check(self.lib.kvc_evict(self._ctx, stream_id), "evict_frames")

    def rollback_frame(self, stream_id: int = 0):
        """Undo the stream's most recent frame (deferred eviction must be on;
        between steps, after plan)."""
        self._check(self.lib.kvc_rollback(self._ctx, stream_id), "rollback_frame")

    def plan(self, stream=None):
        rc = self.lib.kvc_plan(self._ctx, None if self.metadata_only else self._stream(stream))
        self._check(rc, "plan")
        self._planned = True

    def compute_attention(self, block_idx: int, q, out=None, stream=None, no_alloc: bool = False, rope=None):
        """Paged attention of the step's queries q [R, H, D] for one block;
        plans first when called for block 0 of an unplanned step.  no_alloc
        runs kvc_run_no_alloc (split partials in the library's static device
        scratch); out must then be given, since allocating it would defeat
        the purpose.  rope = (cos, sin), float32 [R, D/2] each, turns the
        queries by those angles first (kvc_run_rope)."""
        if block_idx == 0 and not self._planned:
            self.plan(stream)
        rows = q.shape[0]
        self._check_tensor(q, rows, "q")
        if out is None:
            if no_alloc:
                raise KvcError(KVC_ERR_ARG, "no_alloc needs a preallocated out")
            out = self.torch.empty_like(q)
        else:
            self._check_tensor(out, rows, "out")
        if rope is not None:
            if no_alloc:
                raise KvcError(KVC_ERR_ARG, "the rotary embedding runs through the workspace, not no_alloc")
            cp, sp = self._check_tables(rope, rows)
            rc = self.lib.kvc_run_rope(self._ctx, block_idx, q.data_ptr(), cp, sp, out.data_ptr(),
                                       self._stream(stream))
            self._check(rc, "compute_attention")
            return out
        fn = self.lib.kvc_run_no_alloc if no_alloc else self.lib.kvc_run
        rc = fn(self._ctx, block_idx, q.data_ptr(), out.data_ptr(), self._stream(stream))
        self._check(rc, "compute_attention")
        return out

    def append_run(self, block_idx: int, ks, vs, q, out=None, stream=None):
        """kvc_run_append: this step's appends of one block and its attention.
        ks, vs: {stream id: [F*T, H, D] (or [F, T, H, D]) rows} of the planned
        streams; q, out as compute_attention.  Plans first when called for
        block 0 of an unplanned step."""
        if block_idx == 0 and not self._planned:
            self.plan(stream)
        rows = q.shape[0]
        self._check_tensor(q, rows, "q")
        if out is None:
            out = self.torch.empty_like(q)
        else:
            self._check_tensor(out, rows, "out")
        n = self.cfg.num_streams
        kp = (_P * n)()
        vp = (_P * n)()
        T = self.cfg.tokens_per_frame
        for s, kt in ks.items():
            vt = vs[s]
            k2 = kt.reshape(-1, *kt.shape[-2:])
            v2 = vt.reshape(-1, *vt.shape[-2:])
            if k2.shape[0] % T:
                raise KvcError(KVC_ERR_ARG, f"stream {s}: rows not a whole number of frames")
            self._check_tensor(k2, k2.shape[0], "k")
            self._check_tensor(v2, v2.shape[0], "v")
            kp[s] = k2.data_ptr()
            vp[s] = v2.data_ptr()
        rc = self.lib.kvc_run_append(self._ctx, block_idx, kp, vp, q.data_ptr(), out.data_ptr(), self._stream(stream))
        self._check(rc, "append_run")
        return out

    def raw_run_append(self, block_idx: int, k_ptrs, v_ptrs, q_ptr: int, o_ptr: int, hip_stream: int):
        """kvc_run_append on raw addresses: k_ptrs / v_ptrs per stream id
        (num_streams entries, 0 where a stream is not planned)."""
        n = self.cfg.num_streams
        kp = (_P * n)(*k_ptrs)
        vp = (_P * n)(*v_ptrs)
        rc = self.lib.kvc_run_append(self._ctx, block_idx, kp, vp, q_ptr, o_ptr, hip_stream)
        if rc:
            self._check(rc, "append_run")

    def reset(self):
        self._check(self.lib.kvc_reset(self._ctx), "reset")
        self._planned = False

    def get_cache_stats(self, stream_id: int = 0) -> Dict[str, int]:
        s = KvcStats()
        self._check(self.lib.kvc_get_stats(self._ctx, stream_id, ctypes.byref(s)), "get_cache_stats")
        return {"frame_count": s.frame_count, "scale_pages": s.scale_pages, "live_pages": s.live_pages,
                "free_pages": s.free_pages, "special_tokens": s.special_tokens,
                "special_pages": s.special_pages, "free_special_pages": s.free_special_pages}

    def get_plan(self) -> Dict[str, np.ndarray]:
        n = ctypes.c_int32()
        ni = ctypes.c_int32()
        self._check(self.lib.kvc_get_plan(self._ctx, None, None, None, None, None, None, None, 0, 0,
                                          ctypes.byref(n), ctypes.byref(ni)), "get_plan")
        ns, nidx = n.value, ni.value
        arrs = {"planned": np.zeros(ns, np.int32), "kv_indptr": np.zeros(ns + 1, np.int32),
                "kv_indices": np.zeros(max(nidx, 1), np.int32), "last_page_len": np.zeros(ns, np.int32),
                "n_patch_pages": np.zeros(ns, np.int32), "qo_indptr": np.zeros(ns + 1, np.int32),
                "n_splits": np.zeros(ns, np.int32)}
        ptr = {k: v.ctypes.data_as(_PI32) for k, v in arrs.items()}
        self._check(self.lib.kvc_get_plan(self._ctx, ptr["planned"], ptr["kv_indptr"], ptr["kv_indices"],
                                          ptr["last_page_len"], ptr["n_patch_pages"], ptr["qo_indptr"],
                                          ptr["n_splits"], ns, max(nidx, 1), None, None), "get_plan")
        arrs["kv_indices"] = arrs["kv_indices"][:nidx]
        return arrs

    def get_plan_shape(self) -> Dict[str, int]:
        """Attention work-groups of the current plan and query rows per group."""
        items = ctypes.c_int32()
        rows = ctypes.c_int32()
        self._check(self.lib.kvc_get_plan_shape(self._ctx, ctypes.byref(items), ctypes.byref(rows)),
                    "get_plan_shape")
        return {"work_items": items.value, "group_rows": rows.value}

    def get_split_partials(self, stream=None):
        """The split partials of the latest run: (lse [MAX_SPLITS, H, tiles, 32]
        float32 base-2 log-sum-exps, o [MAX_SPLITS, H, tiles, D/32, 4, 64, 4]
        raw 16-bit normalised outputs); see kvc_get_split_partials."""
        nl, no = ctypes.c_int64(), ctypes.c_int64()
        self._check(self.lib.kvc_get_split_partials(self._ctx, None, 0, None, 0, ctypes.byref(nl), ctypes.byref(no),
                                                    None), "get_split_partials")
        lse = np.zeros(nl.value, np.float32)
        o = np.zeros(no.value, np.uint16)
        hs = self._stream(stream)
        self._check(self.lib.kvc_get_split_partials(self._ctx, lse.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                                    lse.size, o.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                                    o.size, ctypes.byref(nl), ctypes.byref(no), hs),
                    "get_split_partials")
        H, D = self.cfg.num_heads, self.cfg.head_dim
        tiles = nl.value // (MAX_SPLITS * H * 32)
        return lse.reshape(MAX_SPLITS, H, tiles, 32), o.reshape(MAX_SPLITS, H, tiles, D // 32, 4, 64, 4)

    def get_plan_image(self) -> np.ndarray:
        """The int32 plan image that kvc_plan uploads for the kernels."""
        n = ctypes.c_int32()
        self._check(self.lib.kvc_get_plan_image(self._ctx, None, 0, ctypes.byref(n)), "get_plan_image")
        buf = np.zeros(max(n.value, 1), np.int32)
        self._check(self.lib.kvc_get_plan_image(self._ctx, buf.ctypes.data_as(_PI32), buf.size, ctypes.byref(n)),
                    "get_plan_image")
        return buf[:n.value]

    def set_option(self, option: int, value: int):
        self._check(self.lib.kvc_set_option(self._ctx, option, value), "set_option")

    def get_option(self, option: int) -> int:
        v = ctypes.c_int64()
        self._check(self.lib.kvc_get_option(self._ctx, option, ctypes.byref(v)), "get_option")
        return v.value

    def profile_read(self, kernel: int, reset: bool = False):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        self._check(self.lib.kvc_profile_read(self._ctx, kernel, ctypes.byref(ms), ctypes.byref(n), int(reset)),
                    "profile_read")
        return ms.value, n.value

    # -- low-overhead calls on raw addresses (no per-call tensor checks) --
    def raw_append(self, block_idx: int, k_ptr: int, v_ptr: int, stream_id: int, hip_stream: int):
        rc = self.lib.kvc_append_frame(self._ctx, stream_id, block_idx, k_ptr, v_ptr, hip_stream)
        if rc:
            self._check(rc, "append_frame")

    def raw_plan(self, hip_stream: int):
        rc = self.lib.kvc_plan(self._ctx, hip_stream)
        if rc:
            self._check(rc, "plan")
        self._planned = True

    def raw_append_frames(self, block_idx: int, k_ptr: int, v_ptr: int, num_frames: int, stream_id: int,
                          hip_stream: int):
        rc = self.lib.kvc_append_frames(self._ctx, stream_id, block_idx, k_ptr, v_ptr, num_frames, hip_stream)
        if rc != KVC_OK:
            self._check(rc, "append_frames")

    def raw_run(self, block_idx: int, q_ptr: int, o_ptr: int, hip_stream: int):
        rc = self.lib.kvc_run(self._ctx, block_idx, q_ptr, o_ptr, hip_stream)
        if rc:
            self._check(rc, "compute_attention")

    def close(self):
        if self._ctx:
            self.lib.kvc_destroy(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
