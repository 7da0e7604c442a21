"""Seeded synthetic inputs for the two-stream paged KV-cache attention.

This module is shared by the CPU oracle and by the HIP path's tests and bench.
It holds none of the method's arithmetic: it only draws numbers, rounds them
to bf16 storage, and describes workload shapes.

Every draw is keyed by (seed, stream, frame, block, tensor, part) through
NumPy's counter-based Philox generator, so any frame of any stream can be
regenerated on demand without storing history (the oracle regenerates the
visible frames of a long stream this way).

The only random numbers the method itself consumes are the initial orders of
the two free lists (patch pages and special pages).  They are drawn here and
passed to both sides as explicit inputs.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}
PART_PATCH = 0
PART_SPECIAL = 1


def _key(seed: int, stream: int, frame: int, block: int, tensor: int, part: int):
    if not (0 <= stream < (1 << 16) and 0 <= frame < (1 << 32) and 0 <= block < (1 << 12)):
        raise ValueError("key field out of range")
    packed = (stream << 48) | (frame << 16) | (block << 4) | (tensor << 1) | part
    return [int(seed) & ((1 << 64) - 1), packed]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite normals here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (numpy's round to nearest even) and
    return the 16-bit patterns as uint16."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# Bit-pattern array type of each element type.
BITS_DTYPE = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}


def bits_to_f32(b: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Exact widening of the bit patterns of the given element type ("bf16",
    "f16" or "f32") to float32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(b)
    if dtype == "f16":
        return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(b, dtype=np.uint32).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def f32_to_bits(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    raise ValueError(f"unknown dtype {dtype}")


def normal_bf16(seed: int, stream: int, frame: int, block: int, tensor: int, part: int,
                shape, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Seeded N(0, scale^2) values rounded to the element type, as bits."""
    g = np.random.Generator(np.random.Philox(key=_key(seed, stream, frame, block, tensor, part)))
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return f32_to_bits(x, dtype)


def special_rows(T: int, n_special: int, special_row_offset: int) -> np.ndarray:
    """Row indices, inside a frame's [T] rows, that hold the special tokens."""
    return np.arange(special_row_offset, special_row_offset + n_special)


def patch_rows(T: int, n_special: int, special_row_offset: int) -> np.ndarray:
    """Row indices of the patch tokens, in order."""
    r = np.arange(T)
    return r[(r < special_row_offset) | (r >= special_row_offset + n_special)]


def frame_tensor(seed: int, stream: int, frame: int, block: int, which: str,
                 T: int, H: int, D: int, n_special: int, special_row_offset: int,
                 scale: float = 1.0, patch_real: bool = True, dtype: str = "bf16") -> np.ndarray:
    """One frame's Q, K or V as bit patterns of `dtype`, shape [T, H, D] (NHD).

    Patch rows and special rows are drawn from separate keys, so the special
    rows of any frame can be regenerated cheaply.  With patch_real=False the
    patch rows are zero (used for frames whose patch page is evicted before
    any checked step, so a long stream need not draw them)."""
    t = TENSOR_IDS[which]
    out = np.zeros((T, H, D), dtype=BITS_DTYPE[dtype])
    pr = patch_rows(T, n_special, special_row_offset)
    sr = special_rows(T, n_special, special_row_offset)
    if patch_real and len(pr):
        out[pr] = normal_bf16(seed, stream, frame, block, t, PART_PATCH, (len(pr), H, D), scale, dtype)
    if len(sr):
        out[sr] = normal_bf16(seed, stream, frame, block, t, PART_SPECIAL, (len(sr), H, D), scale, dtype)
    return out


def special_part(seed: int, stream: int, frame: int, block: int, which: str,
                 n_special: int, H: int, D: int, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Only the special rows of a frame, [n_special, H, D] bits (the same
    values frame_tensor places at the special rows)."""
    return normal_bf16(seed, stream, frame, block, TENSOR_IDS[which], PART_SPECIAL,
                       (n_special, H, D), scale, dtype)


def free_list_order(seed: int, n: int, first_id: int, which: int) -> np.ndarray:
    """Initial order of a free list: the IDs first_id .. first_id+n-1, ascending
    when seed == 0, otherwise a seeded permutation (which=0 patch, 1 special)."""
    ids = np.arange(first_id, first_id + n, dtype=np.int32)
    if seed == 0:
        return ids
    g = np.random.Generator(np.random.Philox(key=[int(seed), (0xF1EE << 16) | which]))
    return ids[g.permutation(n)].astype(np.int32)


def rope_tables(frame0: int, num_frames: int, T: int, D: int, n_special: int, special_row_offset: int,
                base: float = 100.0):
    """Caller-side rotary tables for the rows of frames frame0 ..
    frame0 + num_frames - 1 (global frame indices), as the caller of a
    rotary embedding would build them: float32 cos and sin [num_frames * T,
    D/2].  A stand-in for a 3-D layout: the D/2 pairs are split into three
    bands that turn with the frame index, the patch's row and its column on a
    near-square grid of the frame's patches (special tokens sit at row and
    column 0); band j of size m has frequencies base^(-i/m), i < m.  These are
    inputs, drawn the same way for both sides; no randomness is involved."""
    half = D // 2
    m = half // 3
    sizes = (half - 2 * m, m, m)
    P = T - n_special
    width = max(1, int(np.ceil(np.sqrt(max(P, 1)))))
    rows = np.arange(T)
    is_special = (rows >= special_row_offset) & (rows < special_row_offset + n_special)
    patch_idx = np.where(rows < special_row_offset, rows, rows - n_special)
    py = np.where(is_special, 0, patch_idx // width).astype(np.float64)
    px = np.where(is_special, 0, patch_idx % width).astype(np.float64)
    cos = np.empty((num_frames * T, half), np.float32)
    sin = np.empty_like(cos)
    for f in range(num_frames):
        pos = (np.full(T, float(frame0 + f)), py, px)
        ang = np.concatenate([pos[j][:, None] * base ** (-np.arange(sizes[j]) / max(sizes[j], 1))[None, :]
                              for j in range(3)], axis=1)
        cos[f * T:(f + 1) * T] = np.cos(ang)
        sin[f * T:(f + 1) * T] = np.sin(ang)
    return cos, sin


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic frame stream workload."""
    name: str
    num_blocks: int
    num_heads: int
    head_dim: int
    patch_tokens: int          # P
    num_special_tokens: int    # n_s
    page_size: int             # >= P
    scale_frames: int          # S
    sliding_window: int        # W
    frames: tuple              # frames streamed per stream (history length at the end)
    seed: int
    max_patch_pages: int
    max_special_pages: int
    shuffle_free_lists: bool = False
    special_row_offset: Optional[int] = None   # None: specials after the patches
    dtype: str = "bf16"                         # element type: "bf16", "f16" or "f32"

    @property
    def tokens_per_frame(self) -> int:
        return self.patch_tokens + self.num_special_tokens

    @property
    def num_streams(self) -> int:
        return len(self.frames)

    @property
    def row_offset(self) -> int:
        return self.patch_tokens if self.special_row_offset is None else self.special_row_offset


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _special_pages_for(frames, n_s, pg):
    return sum(_ceil_div(f * n_s, pg) for f in frames)


WORKLOADS: Dict[str, Workload] = {
    # Tiny stream the oracle checks in milliseconds: one spare patch page beyond
    # S+W, so evicted pages are reused at once.
    "tiny": Workload("tiny", 1, 2, 32, 16, 6, 16, 1, 4, (12,), 0,
                     max_patch_pages=1 + 4 + 1, max_special_pages=5),
    # 256 patches + 6 specials per frame, scale 8, window 64, 200 frames.
    "base": Workload("base", 24, 16, 64, 256, 6, 256, 8, 64, (200,), 1,
                     max_patch_pages=88, max_special_pages=_special_pages_for((200,), 6, 256)),
    # 518x378 frames at patch 14: 37x27 = 999 patches in 1024-token pages.
    "r518": Workload("r518", 24, 16, 64, 999, 6, 1024, 8, 64, (500,), 2,
                     max_patch_pages=88, max_special_pages=_special_pages_for((500,), 6, 1024)),
    # 10,000-frame stream: 60,000 special tokens.
    "long": Workload("long", 24, 16, 64, 256, 6, 256, 8, 64, (10000,), 3,
                     max_patch_pages=88, max_special_pages=_special_pages_for((10000,), 6, 256)),
    # Four streams at different history lengths batched into one plan/run,
    # both free lists shuffled.
    "frag": Workload("frag", 24, 8, 128, 256, 6, 256, 4, 32, (50, 400, 1500, 4000), 4,
                     max_patch_pages=4 * (4 + 32 + 1) + 4,
                     max_special_pages=_special_pages_for((50, 400, 1500, 4000), 6, 256),
                     shuffle_free_lists=True),
}


def stream_join_step(wl: Workload, stream: int) -> int:
    """Global step at which a stream starts advancing; all streams end together."""
    return max(wl.frames) - wl.frames[stream]
