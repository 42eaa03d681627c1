"""Reference packing of ragged K/V for variable-length cross-attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): product code never
imports this module.

TensorRT-LLM PR #18973 "FA4 variable-length cross-attention", section Description: two CFG
branches with unequal text lengths pack their K/V into one flat, unpadded buffer, sequence
b's keys being rows [cu_seqlens_kv[b], cu_seqlens_kv[b+1]); Q stays padded. cu_seqlens_kv and
max_seqlen_kv depend only on the length layout and are prepared once per layout (section
Description; section Acceptance criteria). The packing step is a gather/concatenation of each
branch's valid rows (section Acceptance criteria: pack_ragged_kv; section Microbenchmark: its
K/V gather/cat).

Reading taken where the page is silent: a branch's valid rows are its first lens[b] rows of
the padded [B, max_kv, Hkv, D] buffer (the key padding is at the end), and lens[b] = 0 is
allowed by the packing itself (an empty segment), while attention rejects empty segments.
"""
from __future__ import annotations

import numpy as np


def ragged_metadata(lens) -> tuple[np.ndarray, int]:
    """cu_seqlens_kv [B+1] (exclusive prefix sums of lens, int64) and max_seqlen_kv."""
    lens = np.asarray(lens, dtype=np.int64)
    if lens.ndim != 1 or np.any(lens < 0):
        raise ValueError(f"bad lengths {lens.tolist()}")
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    for b in range(lens.shape[0]):
        cu[b + 1] = cu[b] + lens[b]
    return cu, int(lens.max()) if lens.size else 0


def pack_ragged(padded: np.ndarray, lens) -> tuple[np.ndarray, np.ndarray]:
    """Rows [0, lens[b]) of padded[b] for b = 0..B-1, concatenated: ([total, ...], cu)."""
    lens = np.asarray(lens, dtype=np.int64)
    if padded.ndim < 2 or lens.shape != (padded.shape[0],) or np.any(lens > padded.shape[1]):
        raise ValueError(f"lengths {lens.tolist()} do not fit padded {padded.shape}")
    cu, _ = ragged_metadata(lens)
    packed = np.zeros((int(cu[-1]),) + padded.shape[2:], dtype=padded.dtype)
    for b in range(padded.shape[0]):
        packed[cu[b]:cu[b + 1]] = padded[b, :lens[b]]
    return packed, cu
