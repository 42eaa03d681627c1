"""Softmax attention of a query chunk against cached keys/values, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): product code never
imports this module.

What is computed, for one sequence b, query row t and query head h:

    J        = the keys row (b, t, h) may see (rules below)
    s_j      = scale * <q_t, k_j>           for j in J, scale = 1/sqrt(D) by default
    m        = max_j s_j
    p_j      = exp(s_j - m)
    o        = sum_j p_j v_j / sum_j p_j
    lse      = m + log(sum_j p_j)

This is plain two-pass (max-subtracted) softmax attention, the definition that
torch's scaled_dot_product_attention implements; the fish-speech page compares
its active-prefix path against exactly that routine ("perf(text2semantic): pass
only active KV cache prefix to SDPA", sections Problem and Correctness and
compatibility validation). No online/streaming softmax is used here.

Key-set rules:

* Active prefix: only cache rows [0, kv_len) are keys, never the rest of the
  preallocated capacity (fish-speech #1312, section Change). kv_len must
  satisfy 1 <= kv_len <= capacity; 0 and capacity+1 are rejected (fish-speech
  #1312, author's reply listing the valid and invalid bounds).
* Query positions are bottom-right aligned: query t of a chunk of Tq queries
  sits at absolute position p = kv_len - Tq + t. The causal mask is the
  full-length causal mask cut to the active key length (fish-speech #1312,
  section Change); decode (Tq = 1) then sees every active key.
* Masks: NONE (every active key), CAUSAL (j <= p), BLOCK_CAUSAL with block
  size beta (floor(j/beta) <= floor(p/beta); beta = 1 is CAUSAL).
* GQA: query head h reads KV head h // (Hq // Hkv), the head that
  repeat_interleave over the head dimension would have placed there
  (fish-speech #1312, section Problem); no expansion is materialised.
* Packed K/V: sequence b's keys are the rows [cu[b], cu[b+1]) of a packed
  [total, Hkv, D] buffer, Q stays padded (TensorRT-LLM #18973 "FA4
  variable-length cross-attention", section Description). The result must
  equal padded K/V with a key-padding mask (same page, Acceptance criteria).
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_CAUSAL = 2

_ROW_BLOCK = 256  # rows per matmul block; rows are independent, blocking is not a reordering


def default_scale(D: int) -> float:
    """1/sqrt(D), SDPA's default scale (fish-speech #1312 compares against SDPA)."""
    return 1.0 / math.sqrt(D)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: the group index h // (Hq/Hkv)."""
    if Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return h // (Hq // Hkv)


def check_kv_len(kv_len: int, capacity: int) -> None:
    """Reject an active prefix outside [1, capacity] (fish-speech #1312 reply: 1 and
    the capacity are valid, 0 and capacity+1 are not)."""
    if not (1 <= int(kv_len) <= int(capacity)):
        raise ValueError(f"kv_len={kv_len} outside [1, {capacity}]")


def visible_keys(t: int, Tq: int, kv_len: int, mask: int, block: int = 1) -> np.ndarray:
    """Boolean [kv_len]: which of the active keys query t of the chunk may see."""
    p = kv_len - Tq + t
    j = np.arange(kv_len)
    if mask == MASK_NONE:
        return np.ones(kv_len, dtype=bool)
    if mask == MASK_CAUSAL:
        return j <= p
    if mask == MASK_BLOCK_CAUSAL:
        if block < 1:
            raise ValueError("block size must be >= 1")
        return (j // block) <= (p // block) if p >= 0 else np.zeros(kv_len, dtype=bool)
    raise ValueError(f"unknown mask {mask}")


def visibility_matrix(Tq: int, kv_len: int, mask: int, block: int = 1) -> np.ndarray:
    """Boolean [Tq, kv_len] built row by row from ``visible_keys``."""
    return np.stack([visible_keys(t, Tq, kv_len, mask, block) for t in range(Tq)]) if Tq else \
        np.zeros((0, kv_len), dtype=bool)


def active_slices(k_cache: np.ndarray, v_cache: np.ndarray, full_mask: np.ndarray, kv_len: int):
    """The K, V and mask an active-prefix call hands to attention: rows/columns [0, kv_len)
    of the full-capacity tensors (fish-speech #1312, section Change). Returns views."""
    check_kv_len(kv_len, k_cache.shape[0])
    return k_cache[:kv_len], v_cache[:kv_len], full_mask[..., :kv_len]


def _softmax_rows(s: np.ndarray, allowed: np.ndarray):
    """Two-pass softmax of each row of s over the allowed entries. Returns (p, l, m)."""
    if not allowed.any(axis=1).all():
        raise ValueError("a query row has no visible key")
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)  # exp(-inf) = 0 exactly for hidden keys
    l = p.sum(axis=1, keepdims=True)
    return p, l, m


def attend_keys(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray,
                scale: float | None = None):
    """Attention of q [Tq, Hq, D] over the key rows k, v [L, Hkv, D] with a boolean
    visibility matrix allowed [Tq, L] shared by all heads.

    Returns o [Tq, Hq, D] and lse [Hq, Tq], fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    L, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape:
        raise ValueError("q/k/v head dims disagree")
    if allowed.shape != (Tq, L):
        raise ValueError(f"mask shape {allowed.shape} != {(Tq, L)}")
    scale = default_scale(D) if scale is None else float(scale)
    o = np.zeros((Tq, Hq, D), dtype=np.float64)
    lse = np.zeros((Hq, Tq), dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        kg = k[:, g, :]
        vg = v[:, g, :]
        for r0 in range(0, Tq, _ROW_BLOCK):
            r1 = min(Tq, r0 + _ROW_BLOCK)
            s = (q[r0:r1, h, :] @ kg.T) * scale
            p, l, m = _softmax_rows(s, allowed[r0:r1])
            o[r0:r1, h, :] = (p @ vg) / l
            lse[h, r0:r1] = (m + np.log(l))[:, 0]
    return o, lse


def attend_prefix(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, kv_len: int,
                  mask: int = MASK_NONE, block: int = 1, scale: float | None = None):
    """Active-prefix attention for one sequence: q [Tq, Hq, D] against cache rows
    [0, kv_len) of k_cache, v_cache [cap, Hkv, D]."""
    cap = k_cache.shape[0]
    check_kv_len(kv_len, cap)
    Tq = q.shape[0]
    allowed = visibility_matrix(Tq, kv_len, mask, block)
    return attend_keys(q, k_cache[:kv_len], v_cache[:kv_len], allowed, scale)


def attend_full_capacity_masked(q, k_cache, v_cache, kv_len: int, mask: int = MASK_NONE,
                                block: int = 1, scale: float | None = None):
    """The comparison arm: every one of the cap cache rows is a key position and rows
    j >= kv_len are hidden by the mask (fish-speech #1312, section Problem: full-capacity
    K/V with a masked, unpopulated tail)."""
    cap = k_cache.shape[0]
    check_kv_len(kv_len, cap)
    Tq = q.shape[0]
    allowed = np.zeros((Tq, cap), dtype=bool)
    allowed[:, :kv_len] = visibility_matrix(Tq, kv_len, mask, block)
    return attend_keys(q, k_cache, v_cache, allowed, scale)


def attend_batch_prefix(q, k_cache, v_cache, kv_lens, mask: int = MASK_NONE, block: int = 1,
                        scale: float | None = None):
    """Batched active-prefix attention: q [B, Tq, Hq, D], caches [B, cap, Hkv, D],
    kv_lens [B] (one active prefix per sequence). Returns o [B, Tq, Hq, D], lse [B, Hq, Tq]."""
    B = q.shape[0]
    outs = [attend_prefix(q[b], k_cache[b], v_cache[b], int(kv_lens[b]), mask, block, scale)
            for b in range(B)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def attend_packed(q, k_packed, v_packed, cu_seqlens_kv, mask: int = MASK_NONE, block: int = 1,
                  scale: float | None = None):
    """Packed ragged K/V: q [B, Tq, Hq, D] padded, k/v [total, Hkv, D], sequence b's keys
    are rows [cu[b], cu[b+1]) (TensorRT-LLM #18973, section Description)."""
    cu = np.asarray(cu_seqlens_kv, dtype=np.int64)
    B = q.shape[0]
    if cu.shape != (B + 1,) or cu[0] != 0 or np.any(np.diff(cu) <= 0) or cu[-1] != k_packed.shape[0]:
        raise ValueError(f"bad cu_seqlens_kv {cu.tolist()} for total {k_packed.shape[0]}")
    outs = []
    for b in range(B):
        kb = k_packed[cu[b]:cu[b + 1]]
        vb = v_packed[cu[b]:cu[b + 1]]
        outs.append(attend_prefix(q[b], kb, vb, kb.shape[0], mask, block, scale))
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def brute_force(q, k, v, kv_len: int, mask: int = MASK_NONE, block: int = 1,
                scale: float | None = None):
    """Scalar-loop twin of ``attend_prefix`` for tiny shapes: every dot product and sum
    with math.fsum, every exponential with math.exp, every visibility test spelled out."""
    Tq, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if not (1 <= kv_len <= len(k)):
        raise ValueError("kv_len out of range")
    o = [[[0.0] * D for _ in range(Hq)] for _ in range(Tq)]
    lse = [[0.0] * Tq for _ in range(Hq)]
    for t in range(Tq):
        pos = kv_len - Tq + t
        for h in range(Hq):
            g = h // group
            scores = []
            for j in range(kv_len):
                if mask == MASK_CAUSAL and j > pos:
                    continue
                if mask == MASK_BLOCK_CAUSAL and (pos < 0 or j // block > pos // block):
                    continue
                s = scale * math.fsum(float(q[t][h][d]) * float(k[j][g][d]) for d in range(D))
                scores.append((j, s))
            if not scores:
                raise ValueError("a query row has no visible key")
            m = max(s for _, s in scores)
            w = [(j, math.exp(s - m)) for j, s in scores]
            den = math.fsum(p for _, p in w)
            for d in range(D):
                o[t][h][d] = math.fsum(p * float(v[j][g][d]) for j, p in w) / den
            lse[h][t] = m + math.log(den)
    return np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64)


def flops(Tq: int, kv_len: int, Hq: int, D: int, mask: int = MASK_NONE, block: int = 1) -> int:
    """Algorithmic flops of one sequence's attention: 4*D per visible (query, key, head)
    triple (QK^T and PV multiply-adds; the exponentials are not counted)."""
    pairs = int(visibility_matrix(Tq, kv_len, mask, block).sum())
    return 4 * D * Hq * pairs
