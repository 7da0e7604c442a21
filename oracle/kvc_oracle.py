"""CPU oracle for the two-stream paged KV-cache prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library; the only module both sides use is
the seeded input generator `kvc_synth`, which holds none of the arithmetic
below.

It is deliberately plain and slow: Python deques for the allocator, NumPy
arrays for a simulated page pool, and a dense float64 softmax attention over
the visible tokens.  Every function cites the passage it follows.  Sources are
five web pages about the lingbot-map paged KV cache; they are cited by a short
tag and a section name:

  [p1] "How FlashInfer KV Cache Attention Accelerates Streaming 3D
       Reconstruction Over SDPA"
  [p2] "How LingBot-Map Uses FlashInfer KV Cache for Streaming 3D
       Reconstruction"
  [p3] "How FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in
       Streaming Inference"
  [p4] "FlashInfer Backend in LingBot-Map: Accelerating Streaming Inference
       with Paged KV Cache"
  [p5] "How Paged KV Cache Attention Achieves Stable Inference in Ling-Bot-Map"

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * softmax scale 1/sqrt(D) (the dense-attention check path of [p2]
    §Attention Kernel Execution uses PyTorch's default scale);
  * free lists are FIFO: pages are taken from the left and freed to the right;
  * the live window includes the current frame, and the first S frames are the
    scale frames, so frame f is visible at step t iff f < S or f > t - W;
  * the last page length lies in [1, page_size] (a full tail page counts as
    page_size, never 0);
  * special tokens of a frame occupy rows [special_row_offset,
    special_row_offset + n_s) of its [T, H, D] tensors, patch rows are the rest
    in order;
  * patch pages padded beyond P slots ([p2] §Physical Memory Layout) are
    excluded from the softmax by length, never attended as zero keys;
  * several streams share one pool per block and one pair of free lists and
    advance in ascending stream order inside a step; each stream attends only
    to its own pages (batch-prefill semantics of [p1] §Plan Reuse and Kernel
    Optimization);
  * the rotary embedding turns interleaved pairs (2i, 2i+1) of each head by
    angles from caller-supplied cos/sin tables [T, D/2] (the pages give no
    frequencies), computed in float64 and rounded once to the element type.

Parity pins: every function here is pinned by the CPU tests (worked example of
[p3] §Inspecting Cache Statistics, closed forms, invariants, PyTorch's
scaled_dot_product_attention and logsumexp as second routines, brute force on
tiny inputs, the split-KV merge identity, paged-vs-dense identity and page-ID
permutation invariance; for the rotary embedding: brute-force nearest
rounding, the identity and quarter-turn rotations, complex multiplication,
norm preservation, composition and the relative-position identity), and planted mistakes in each are caught by some pin.
"""
from __future__ import annotations

import collections
import dataclasses
import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from kvc_synth import BITS_DTYPE, bits_to_f32, patch_rows, special_rows


@dataclasses.dataclass
class OracleConfig:
    num_heads: int
    head_dim: int
    tokens_per_frame: int          # T = P + n_s
    num_special_tokens: int        # n_s
    page_size: int                 # pg >= P
    scale_frames: int              # S
    sliding_window: int            # W
    max_patch_pages: int
    max_special_pages: int
    num_streams: int = 1
    special_row_offset: Optional[int] = None   # None: specials after patches
    dtype: str = "bf16"                        # element type of K, V, Q: "bf16", "f16" or "f32"

    @property
    def patch_tokens(self) -> int:
        return self.tokens_per_frame - self.num_special_tokens

    @property
    def row_offset(self) -> int:
        return self.patch_tokens if self.special_row_offset is None else self.special_row_offset

    @property
    def max_num_pages(self) -> int:
        # [p2] §Physical Memory Layout: max_num_pages = max_patch_pages + max_special_pages
        return self.max_patch_pages + self.max_special_pages


class PoolExhausted(RuntimeError):
    pass


@dataclasses.dataclass
class FrameSlots:
    """Where one frame's tokens go: its patch page, and one (page, slot) per
    special token."""
    patch_page: int
    special: List[Tuple[int, int]]


@dataclasses.dataclass
class _StreamState:
    scale_patch_pages: List[int]
    live_window_patch_pages: collections.deque
    all_special_pages: List[int]
    special_tokens: int
    frame_count: int
    frames: List[FrameSlots]
    # deferred eviction: window pages evicted since the last append (oldest
    # first), out of the table but not yet free
    held_back: List[int] = dataclasses.field(default_factory=list)
    undoable: bool = False


class AllocatorReplay:
    """The page bookkeeping of the two-stream cache.

    [p1] §Two-Stream Design for Token Types: patch pages are recyclable and
    managed with deques (free, scale, live window); special pages are
    append-only and never evicted.  [p2] §Patch Stream and Special Stream:
    patch page IDs are [0, max_patch_pages), special IDs
    [max_patch_pages, max_num_pages).  [p3] §Two-Stream Design: a frame takes
    exactly one patch page; special tokens pack continuously across pages,
    a new special page being taken from the free special list when the tail
    page is full.
    """

    def __init__(self, cfg: OracleConfig,
                 free_patch_order: Optional[Sequence[int]] = None,
                 free_special_order: Optional[Sequence[int]] = None):
        self.cfg = cfg
        self._init_patch = list(range(cfg.max_patch_pages)) if free_patch_order is None \
            else [int(x) for x in free_patch_order]
        self._init_special = list(range(cfg.max_patch_pages, cfg.max_num_pages)) \
            if free_special_order is None else [int(x) for x in free_special_order]
        assert sorted(self._init_patch) == list(range(cfg.max_patch_pages))
        assert sorted(self._init_special) == list(range(cfg.max_patch_pages, cfg.max_num_pages))
        # [p2] §Scale Frames vs Sliding Window mentions deferred eviction for
        # frame rollback (key-frame selection) without its rules; the reading
        # used here: evicted window pages are held back until the stream's
        # next append, and only the latest frame can be undone, once.
        self.defer_eviction = False
        self.reset()

    def reset(self):
        """[p5] §Resetting for New Sequences: clear the lists and counters, keep
        the page buffers."""
        self.free_patch_pages = collections.deque(self._init_patch)
        self.free_special_pages = collections.deque(self._init_special)
        self.streams = [
            _StreamState([], collections.deque(), [], 0, 0, [])
            for _ in range(self.cfg.num_streams)
        ]

    def append_frame(self, stream: int) -> FrameSlots:
        """Allocation half of append_frame ([p5] §Frame Appending Without
        Dispatch Overhead; [p3] §Two-Stream Design).

        One free patch page receives the frame's patch tokens; it joins the
        scale pages while fewer than S exist ([p2] §Patch Stream and Special
        Stream: the first scale_frames pages are kept permanently), otherwise
        the live window.  Each special token goes to the next slot of the
        special stream."""
        cfg = self.cfg
        st = self.streams[stream]
        pg = cfg.page_size
        # special pages needed for this frame's tokens
        need = 0
        n = st.special_tokens
        for _ in range(cfg.num_special_tokens):
            if n % pg == 0:
                need += 1
            n += 1
        if need > len(self.free_special_pages):
            raise PoolExhausted("special pool exhausted")
        if not self.free_patch_pages and not st.held_back:
            raise PoolExhausted("no free patch page")
        # the previous frame becomes final: its held-back pages are freed
        self.free_patch_pages.extend(st.held_back)
        st.held_back = []
        page = self.free_patch_pages.popleft()
        if len(st.scale_patch_pages) < cfg.scale_frames:
            st.scale_patch_pages.append(page)
        else:
            st.live_window_patch_pages.append(page)
        slots = []
        for _ in range(cfg.num_special_tokens):
            if st.special_tokens % pg == 0:
                st.all_special_pages.append(self.free_special_pages.popleft())
            slots.append((st.all_special_pages[-1], st.special_tokens % pg))
            st.special_tokens += 1
        st.frame_count += 1
        fs = FrameSlots(page, slots)
        st.frames.append(fs)
        st.undoable = True
        return fs

    def rollback_frame(self, stream: int) -> FrameSlots:
        """Undo the latest frame of the stream (deferred eviction only): the
        page lists return to what they were before that frame's append, with
        the pages it took back at the front of the free lists, and the
        held-back window pages back at the front of the window until the
        window is full again."""
        st = self.streams[stream]
        if not self.defer_eviction or not st.undoable or not st.frames:
            raise RuntimeError("nothing to roll back")
        fs = st.frames.pop()
        opened = sorted({p for p, slot in fs.special if slot == 0}, key=st.all_special_pages.index)
        for p in reversed(opened):
            assert st.all_special_pages[-1] == p
            st.all_special_pages.pop()
            self.free_special_pages.appendleft(p)
        st.special_tokens -= len(fs.special)
        if st.live_window_patch_pages and st.live_window_patch_pages[-1] == fs.patch_page:
            st.live_window_patch_pages.pop()
        else:
            assert st.scale_patch_pages[-1] == fs.patch_page
            st.scale_patch_pages.pop()
        self.free_patch_pages.appendleft(fs.patch_page)
        while st.held_back and len(st.live_window_patch_pages) < self.cfg.sliding_window:
            st.live_window_patch_pages.appendleft(st.held_back.pop())
        st.frame_count -= 1
        st.undoable = False
        return fs

    def evict_frames(self, stream: int) -> List[int]:
        """[p5] §Sliding-Window Eviction Strategy; [p1] FAQ on eviction: live
        window pages beyond the window move back to the free list; scale pages
        stay.  Only page IDs move."""
        st = self.streams[stream]
        freed = []
        while len(st.live_window_patch_pages) > self.cfg.sliding_window:
            p = st.live_window_patch_pages.popleft()
            if self.defer_eviction:
                st.held_back.append(p)
            else:
                self.free_patch_pages.append(p)
            freed.append(p)
        return freed

    def build_visible_page_table(self, stream: int) -> List[int]:
        """[p2] §Page Table Planning and Reuse: scale -> window -> specials."""
        st = self.streams[stream]
        return list(st.scale_patch_pages) + list(st.live_window_patch_pages) + list(st.all_special_pages)

    def compute_last_page_len(self, stream: int) -> int:
        """[p5] §Kernel Dispatch and Sequence Lengths: valid tokens on the final
        page.  With specials, the final page is the tail special page and holds
        the special tokens not on the full pages before it; without specials it
        is a patch page holding P tokens."""
        st = self.streams[stream]
        if st.all_special_pages:
            return st.special_tokens - self.cfg.page_size * (len(st.all_special_pages) - 1)
        return self.cfg.patch_tokens

    def plan(self, streams: Sequence[int], frames: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
        """The per-step plan for the given streams, concatenated in the given
        order ([p3] §Plan-Run Execution Workflow).  frames[i] is the number of
        frames stream i appended this step (default 1): the scale phase takes
        several initialization frames in one pass ([p2] §Frame Processing
        Loop), so the step's queries are all of those frames' rows."""
        if frames is None:
            frames = [1] * len(streams)
        indptr = [0]
        indices: List[int] = []
        last = []
        n_patch = []
        n_special = []
        qo = [0]
        for s, nf in zip(streams, frames):
            tbl = self.build_visible_page_table(s)
            indices += tbl
            indptr.append(len(indices))
            last.append(self.compute_last_page_len(s))
            st = self.streams[s]
            n_patch.append(len(st.scale_patch_pages) + len(st.live_window_patch_pages))
            n_special.append(len(st.all_special_pages))
            qo.append(qo[-1] + nf * self.cfg.tokens_per_frame)
        return {
            "kv_indptr": np.array(indptr, dtype=np.int32),
            "kv_indices": np.array(indices, dtype=np.int32),
            "last_page_len": np.array(last, dtype=np.int32),
            "qo_indptr": np.array(qo, dtype=np.int32),
            "n_patch_pages": np.array(n_patch, dtype=np.int32),
            "n_special_pages": np.array(n_special, dtype=np.int32),
        }

    def get_cache_stats(self, stream: int = 0) -> Dict[str, int]:
        """[p3] §Inspecting Cache Statistics: the five counters."""
        st = self.streams[stream]
        return {
            "frame_count": st.frame_count,
            "scale_pages": len(st.scale_patch_pages),
            "live_pages": len(st.live_window_patch_pages),
            "free_pages": len(self.free_patch_pages),
            "special_tokens": st.special_tokens,
        }


class SimulatedPool:
    """One block's page pool [max_num_pages, 2, page_size, H, D] of element
    bit patterns (uint16 for bf16 and f16, uint32 for f32) ([p1] §Paged KV
    Cache Memory Layout; [p5] §Core Implementation
    Mechanics: dimension 1 is 0 = K, 1 = V; NHD inside a page), zero at start."""

    def __init__(self, cfg: OracleConfig):
        self.cfg = cfg
        self.data = np.zeros((cfg.max_num_pages, 2, cfg.page_size, cfg.num_heads, cfg.head_dim),
                             dtype=BITS_DTYPE[cfg.dtype])

    def write_frame(self, slots: FrameSlots, k_bits: np.ndarray, v_bits: np.ndarray):
        """[p5] §Frame Appending Without Dispatch Overhead: patch rows go to the
        frame's page by slice assignment; special rows to their stream slots."""
        cfg = self.cfg
        pr = patch_rows(cfg.tokens_per_frame, cfg.num_special_tokens, cfg.row_offset)
        sr = special_rows(cfg.tokens_per_frame, cfg.num_special_tokens, cfg.row_offset)
        P = len(pr)
        self.data[slots.patch_page, 0, :P] = k_bits[pr]
        self.data[slots.patch_page, 1, :P] = v_bits[pr]
        for j, (page, slot) in enumerate(slots.special):
            self.data[page, 0, slot] = k_bits[sr[j]]
            self.data[page, 1, slot] = v_bits[sr[j]]


def visible_frames(t: int, scale_frames: int, sliding_window: int) -> List[int]:
    """Frames whose patch tokens are visible at step t (0-based, current frame
    included), written from the definition rather than from the deques: the
    first S frames are permanent ([p2] §Scale Frames vs Sliding Window) and the
    window keeps the W most recent non-scale frames."""
    return [f for f in range(t + 1) if f < scale_frames or f > t - sliding_window]


def gather_dense(cfg: OracleConfig, t: int,
                 frame_kv: Callable[[int], Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Dense history of one stream at step t: patch rows of the visible frames
    in frame order, then the special rows of every frame 0..t in (frame, token)
    order ([p1] §Dense Memory Layout and Linear Scaling describes the dense
    history; [p2] FAQ: specials are never removed)."""
    pr = patch_rows(cfg.tokens_per_frame, cfg.num_special_tokens, cfg.row_offset)
    sr = special_rows(cfg.tokens_per_frame, cfg.num_special_tokens, cfg.row_offset)
    ks, vs = [], []
    for f in visible_frames(t, cfg.scale_frames, cfg.sliding_window):
        k, v = frame_kv(f)
        ks.append(k[pr])
        vs.append(v[pr])
    for f in range(t + 1):
        k, v = frame_kv(f)
        ks.append(k[sr])
        vs.append(v[sr])
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def gather_paged(cfg: OracleConfig, pool: SimulatedPool, plan: Dict[str, np.ndarray],
                 i: int) -> Tuple[np.ndarray, np.ndarray]:
    """The i-th planned stream's visible K and V read through its page table:
    patch pages hold P valid tokens, interior special pages page_size, the last
    page last_page_len ([p1] §Efficient Attention Masking and Padding; [p5]
    §Kernel Dispatch and Sequence Lengths)."""
    lo, hi = plan["kv_indptr"][i], plan["kv_indptr"][i + 1]
    pages = plan["kv_indices"][lo:hi]
    n_patch = int(plan["n_patch_pages"][i])
    last = int(plan["last_page_len"][i])
    ks, vs = [], []
    for j, page in enumerate(pages):
        if j < n_patch:
            n = cfg.patch_tokens
            if j == len(pages) - 1:
                n = last
        elif j == len(pages) - 1:
            n = last
        else:
            n = cfg.page_size
        ks.append(pool.data[page, 0, :n])
        vs.append(pool.data[page, 1, :n])
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def attention_fp64(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Unmasked softmax attention of every query row over every given key,
    per head, in float64 from the exact input values (bf16; f16, the 16-bit
    float the paged kernels also take natively, [p3] §Precision and Hardware
    Utilization; or f32, the full-precision pool of [p3] FAQ on fp32 and [p4]
    §Memory Management and Debugging):
    O = softmax(Q K^T / sqrt(D)) V  ([p1] §Efficient Attention Masking and
    Padding: no boolean mask; [p5] §Kernel Dispatch and Sequence Lengths:
    exact weights over the valid tokens).

    q_bits [T, H, D], k_bits and v_bits [L, H, D] (bit patterns of dtype).
    Returns [T, H, D] float64."""
    q = bits_to_f32(q_bits, dtype).astype(np.float64)
    k = bits_to_f32(k_bits, dtype).astype(np.float64)
    v = bits_to_f32(v_bits, dtype).astype(np.float64)
    T, H, D = q.shape
    out = np.empty((T, H, D), dtype=np.float64)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale          # [T, L]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def lse_base2_fp64(q_bits: np.ndarray, k_bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """log2 of sum_j exp(q.k_j / sqrt(D)) per query row and head, [T, H]: the
    normaliser of the softmax over the given keys, in base 2.  Attention over
    chunks of the keys, each weighted by 2^(lse_chunk - lse_all), sums to the
    attention over all of them, which is what a split-KV partial result must
    carry ([p5] §Kernel Dispatch and Sequence Lengths: exact weights over the
    valid tokens, whatever the split)."""
    q = bits_to_f32(q_bits, dtype).astype(np.float64)
    k = bits_to_f32(k_bits, dtype).astype(np.float64)
    T, H, D = q.shape
    out = np.empty((T, H), dtype=np.float64)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(D)
        m = s.max(axis=1)
        out[:, h] = (m + np.log(np.exp(s - m[:, None]).sum(axis=1))) / math.log(2.0)
    return out


def round_to_elem(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """float64 values rounded to the nearest value of the element type (ties
    to even), as bit patterns (uint16; uint32 for f32).  bf16: 8 significant
    bits and the float32 exponent range; the values here are finite and, when
    non-zero, normal."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "f32":
        return x.astype(np.float32).view(np.uint32)
    m, e = np.frexp(x)                                  # x = m 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) * np.exp2(e.astype(np.float64) - 8.0)   # 8 significant bits, ties to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rope_rotate_fp64(x_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Rotary position embedding applied to query or key rows before they
    enter the cache ([p2] "How LingBot-Map Uses FlashInfer KV Cache for
    Streaming 3D Reconstruction" §3D RoPE Position Encoding and its FAQ on
    temporal information: positions are baked into q and k, so attention
    needs no position lookup).  The pages name a 3-D rotary embedding but give
    no frequency definition, so the angles are the caller's: cos and sin
    [T, D/2] hold, for row t and pair i, the cosine and sine of the angle by
    which elements (2i, 2i+1) of every head of that row turn (the pair read
    as one complex number, multiplied by cos + i sin):
        (a, b) -> (a cos - b sin, a sin + b cos),
    in float64 from the exact 16-bit inputs and the tables' values.
    x_bits [T, H, D]; returns float64 [T, H, D], not rounded."""
    x = bits_to_f32(x_bits, dtype).astype(np.float64)
    T, H, D = x.shape
    c = np.asarray(cos, dtype=np.float64).reshape(T, 1, D // 2)
    s = np.asarray(sin, dtype=np.float64).reshape(T, 1, D // 2)
    a, b = x[:, :, 0::2], x[:, :, 1::2]
    out = np.empty_like(x)
    out[:, :, 0::2] = a * c - b * s
    out[:, :, 1::2] = a * s + b * c
    return out


def rope_fp64(x_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """The rotated rows as they are stored: rope_rotate_fp64 rounded once to
    the element type.  Returns bit patterns [T, H, D]."""
    return round_to_elem(rope_rotate_fp64(x_bits, cos, sin, dtype), dtype)


def pool_bytes(cfg: OracleConfig, num_blocks: int) -> int:
    """Bytes of all block pools: fixed at construction, independent of stream
    length ([p5] FAQ on the sliding window and memory exhaustion)."""
    return num_blocks * cfg.max_num_pages * 2 * cfg.page_size * cfg.num_heads * cfg.head_dim * 2


class OracleStream:
    """Convenience driver: one allocator, simulated pools for selected blocks,
    and the order of calls of one streaming step ([p1] §FlashInferAttention
    Forward Pass: append, evict, then attention with the shared plan)."""

    def __init__(self, cfg: OracleConfig, blocks: Sequence[int] = (0,),
                 free_patch_order=None, free_special_order=None):
        self.cfg = cfg
        self.alloc = AllocatorReplay(cfg, free_patch_order, free_special_order)
        self.pools = {b: SimulatedPool(cfg) for b in blocks}

    def step(self, streams: Sequence[int],
             frame_kv: Callable[[int, int, int], Tuple[np.ndarray, np.ndarray]],
             evict: bool = True, frames: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
        """Advance the given streams by frames[i] frames each (default one;
        several in a scale-phase step, [p2] §Frame Processing Loop).
        frame_kv(stream, frame, block) returns that frame's K and V bits.
        Returns the step's plan."""
        if frames is None:
            frames = [1] * len(streams)
        for s, nf in zip(streams, frames):
            for _ in range(nf):
                f = self.alloc.streams[s].frame_count
                slots = self.alloc.append_frame(s)
                for b, pool in self.pools.items():
                    k, v = frame_kv(s, f, b)
                    pool.write_frame(slots, k, v)
        if evict:
            for s in streams:
                self.alloc.evict_frames(s)
        return self.alloc.plan(streams, frames)

    def attend(self, plan: Dict[str, np.ndarray], block: int, q_bits: np.ndarray) -> np.ndarray:
        """Paged attention of the step: q_bits rows in plan order, stream i's
        at [qo_indptr[i], qo_indptr[i+1])."""
        qo = plan["qo_indptr"]
        outs = []
        for i in range(len(plan["last_page_len"])):
            k, v = gather_paged(self.cfg, self.pools[block], plan, i)
            outs.append(attention_fp64(q_bits[qo[i]:qo[i + 1]], k, v, self.cfg.dtype))
        return np.concatenate(outs, axis=0)
