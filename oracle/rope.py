"""Rotary position embedding applied to keys before they are stored.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): product code never
imports this module.

The streaming-cache page (flashdreams issue #763 "add an opt-in circular KV
policy for streaming attention", section proposed boundary) states that keys
are rotated at their absolute positions before the cache write, which is what
lets a circular buffer hold them in physical order. It prints no RoPE formula.
The reading taken here:

* 1-D rotary embedding: coordinate pairs (a, b) of each key row are rotated by
  the angle theta = position * inv_freq[i] of their pair index i, i.e.
  (a, b) -> (a cos theta - b sin theta, a sin theta + b cos theta);
* the per-pair frequencies inv_freq[0 .. D/2) are the caller's (any base or
  scaling scheme is a choice of that table);
* two pair layouts: "half" pairs coordinate i with i + D/2, "interleaved"
  pairs 2i with 2i + 1;
* the position of a key is its absolute token index: the slab row it is
  written to (index_copy's index), or, in the ring, chunk_id * C + t for row t
  of the chunk_id-th chunk reserved since the last reset;
* arithmetic in fp64 (angle, sine, cosine, the two products and their sum),
  then rounded to fp32 and from fp32 to the cache dtype, round-to-nearest-even
  at each step.
"""
from __future__ import annotations

import numpy as np

LAYOUT_HALF = 0
LAYOUT_INTERLEAVED = 1


def pair_indices(D: int, layout: int) -> tuple[np.ndarray, np.ndarray]:
    """Coordinates (first, second) of the D/2 rotated pairs of a row of length D."""
    if D % 2:
        raise ValueError("D must be even")
    i = np.arange(D // 2)
    if layout == LAYOUT_HALF:
        return i, i + D // 2
    if layout == LAYOUT_INTERLEAVED:
        return 2 * i, 2 * i + 1
    raise ValueError(f"unknown layout {layout}")


def rope_rotate(x: np.ndarray, positions, inv_freq: np.ndarray, layout: int) -> np.ndarray:
    """Rotate rows of x [..., T, H, D] (fp64 values) at positions[T], exact fp64 arithmetic."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    first, second = pair_indices(D, layout)
    pos = np.asarray(positions, dtype=np.int64).astype(np.float64)
    theta = pos[:, None] * np.asarray(inv_freq, dtype=np.float64)[None, :]  # [T, D/2]
    c = np.cos(theta)[:, None, :]  # broadcast over heads
    s = np.sin(theta)[:, None, :]
    a = x[..., first]
    b = x[..., second]
    out = x.copy()
    out[..., first] = a * c - b * s
    out[..., second] = a * s + b * c
    return out


def _f32_to_bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest, ties to even), returned as fp64 values."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(x32)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def round_cache(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> cache dtype (RNE); values returned as fp64."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype == "bf16":
        return _f32_to_bf16_rne(x32)
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def rope_keys(x: np.ndarray, positions, inv_freq: np.ndarray, layout: int, dtype: str) -> np.ndarray:
    """What a fused rotate-then-write stores: rope_rotate rounded to the cache dtype."""
    return round_cache(rope_rotate(x, positions, inv_freq, layout), dtype)


def ring_positions(chunk_id: int, C: int) -> np.ndarray:
    """Absolute positions of the rows of the chunk_id-th chunk reserved since reset."""
    return chunk_id * C + np.arange(C)
