"""Pins of the fp64 attention oracle against things other than itself: scalar brute
force, torch's CPU fp64 scaled_dot_product_attention with an independently built
mask, closed forms, the pages' printed fixture values, and invariants. The last
group plants plausible mistakes into the oracle and checks a pin catches each."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def rnd(*shape):
    return rng.standard_normal(shape)


def sdpa_ref(q, k, v, allowed, scale=None):
    """torch CPU fp64 SDPA over explicitly expanded KV heads (the repeat_interleave
    the library avoids) with a boolean mask [Tq, L]."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, Tq, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    m = torch.from_numpy(allowed)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()


def torch_mask(Tq, L, mask, block=1):
    """Bottom-right aligned masks built from torch primitives, not from the oracle."""
    if mask == A.MASK_NONE:
        return np.ones((Tq, L), dtype=bool)
    if mask == A.MASK_CAUSAL:
        return torch.ones(Tq, L, dtype=torch.bool).tril(diagonal=L - Tq).numpy()
    pos = torch.arange(L - Tq, L)[:, None]
    key = torch.arange(L)[None, :]
    return (torch.div(key, block, rounding_mode="floor")
            <= torch.div(pos, block, rounding_mode="floor")).numpy()


CASES = [
    # Tq, kv_len, cap, Hq, Hkv, D, mask, block
    (1, 1, 4, 2, 1, 8, A.MASK_NONE, 1),
    (3, 7, 9, 4, 2, 8, A.MASK_NONE, 1),
    (3, 7, 9, 4, 2, 8, A.MASK_CAUSAL, 1),
    (5, 5, 6, 4, 4, 4, A.MASK_CAUSAL, 1),
    (4, 11, 12, 6, 2, 4, A.MASK_BLOCK_CAUSAL, 2),
    (4, 11, 12, 6, 2, 4, A.MASK_BLOCK_CAUSAL, 3),
    (2, 9, 16, 8, 2, 16, A.MASK_BLOCK_CAUSAL, 4),
]


@pytest.mark.parametrize("case", CASES)
def test_vectorized_matches_brute_force(case):
    Tq, kv_len, cap, Hq, Hkv, D, mask, block = case
    q, k, v = rnd(Tq, Hq, D), rnd(cap, Hkv, D), rnd(cap, Hkv, D)
    o, lse = A.attend_prefix(q, k, v, kv_len, mask, block)
    ob, lseb = A.brute_force(q.tolist(), k.tolist(), v.tolist(), kv_len, mask, block)
    assert np.max(np.abs(o - ob)) <= 1e-13
    assert np.max(np.abs(lse - lseb)) <= 1e-13


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_sdpa(case):
    Tq, kv_len, cap, Hq, Hkv, D, mask, block = case
    q, k, v = rnd(Tq, Hq, D), rnd(cap, Hkv, D), rnd(cap, Hkv, D)
    o, _ = A.attend_prefix(q, k, v, kv_len, mask, block)
    ref = sdpa_ref(q, k[:kv_len], v[:kv_len], torch_mask(Tq, kv_len, mask, block))
    assert np.max(np.abs(o - ref)) <= 1e-13


def test_lse_matches_logsumexp():
    q, k, v = rnd(4, 4, 8), rnd(10, 2, 8), rnd(10, 2, 8)
    _, lse = A.attend_prefix(q, k, v, 10, A.MASK_CAUSAL)
    allowed = torch_mask(4, 10, A.MASK_CAUSAL)
    for h in range(4):
        s = torch.from_numpy(q[:, h] @ k[:, h // 2].T / math.sqrt(8))
        s = s.masked_fill(~torch.from_numpy(allowed), -math.inf)
        assert np.max(np.abs(torch.logsumexp(s, dim=1).numpy() - lse[h])) <= 1e-13


def test_closed_form_single_key():
    q, k, v = rnd(3, 4, 8), rnd(5, 2, 8), rnd(5, 2, 8)
    o, lse = A.attend_prefix(q, k, v, 1)
    for h in range(4):
        np.testing.assert_array_equal(o[:, h], np.broadcast_to(v[0, h // 2], (3, 8)))
        np.testing.assert_allclose(lse[h], q[:, h] @ k[0, h // 2] / math.sqrt(8), rtol=0, atol=1e-14)


def test_closed_form_identical_keys_is_mean_of_values():
    q, v = rnd(2, 2, 8), rnd(6, 1, 8)
    k = np.repeat(rnd(1, 1, 8), 6, axis=0)
    o, lse = A.attend_prefix(q, k, v, 6)
    np.testing.assert_allclose(o[:, 0], np.broadcast_to(v[:, 0].mean(0), (2, 8)), atol=1e-14)
    np.testing.assert_allclose(lse[0], q[:, 0] @ k[0, 0] / math.sqrt(8) + math.log(6), atol=1e-13)
    o0, _ = A.attend_prefix(np.zeros((1, 1, 8)), rnd(6, 1, 8), v, 6)
    np.testing.assert_allclose(o0[0, 0], v[:, 0].mean(0), atol=1e-14)


def test_closed_form_constant_values_and_dominant_key():
    q, k = rnd(3, 2, 8), rnd(7, 2, 8)
    v = np.full((7, 2, 8), 0.375)
    o, _ = A.attend_prefix(q, k, v, 7)
    np.testing.assert_allclose(o, 0.375, atol=1e-15)
    # one key aligned with q and scaled up dominates the softmax
    q1 = rnd(1, 1, 8)
    k1 = rnd(5, 1, 8)
    k1[3, 0] = 200.0 * q1[0, 0]
    v1 = rnd(5, 1, 8)
    o1, _ = A.attend_prefix(q1, k1, v1, 5)
    np.testing.assert_allclose(o1[0, 0], v1[3, 0], atol=1e-12)


def test_decode_sees_every_active_key():
    """Tq = 1 with the causal mask cut to kv_len is unmasked attention."""
    q, k, v = rnd(1, 4, 8), rnd(9, 2, 8), rnd(9, 2, 8)
    oc, _ = A.attend_prefix(q, k, v, 6, A.MASK_CAUSAL)
    on, _ = A.attend_prefix(q, k, v, 6, A.MASK_NONE)
    np.testing.assert_array_equal(oc, on)


def test_active_prefix_equals_full_capacity_masked_tail():
    """fish-speech #1312, Correctness and compatibility validation: active-prefix attention
    equals full-cache attention with the unpopulated tail masked."""
    for mask, block in [(A.MASK_NONE, 1), (A.MASK_CAUSAL, 1), (A.MASK_BLOCK_CAUSAL, 4)]:
        q, k, v = rnd(5, 4, 16), rnd(32, 2, 16), rnd(32, 2, 16)
        o, lse = A.attend_prefix(q, k, v, 13, mask, block)
        of, lsef = A.attend_full_capacity_masked(q, k, v, 13, mask, block)
        assert np.max(np.abs(o - of)) <= 1e-15
        assert np.max(np.abs(lse - lsef)) <= 1e-14


def test_golden_fp32_active_vs_full_within_page_tolerance():
    """The page's fp32 fixture tolerance (rtol 1e-5, atol 1e-6) holds for the oracle's
    definition evaluated in torch fp32."""
    g = json.load(open(os.path.join(GOLDEN, "active_kv_progression.json")))
    q = torch.from_numpy(rnd(2, 3, 16)).float().permute(1, 0, 2)
    k = torch.from_numpy(rnd(8, 3, 16)).float().permute(1, 0, 2)
    v = torch.from_numpy(rnd(8, 3, 16)).float().permute(1, 0, 2)
    kv_len = 5
    act = torch.nn.functional.scaled_dot_product_attention(q, k[:, :kv_len], v[:, :kv_len])
    m = torch.zeros(2, 8, dtype=torch.bool)
    m[:, :kv_len] = True
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)
    torch.testing.assert_close(act, full, rtol=g["fp32_rtol"], atol=g["fp32_atol"])
    o, _ = A.attend_prefix(q.permute(1, 0, 2).double().numpy(), k.permute(1, 0, 2).double().numpy(),
                           v.permute(1, 0, 2).double().numpy(), kv_len)
    np.testing.assert_allclose(o, act.permute(1, 0, 2).double().numpy(), rtol=g["fp32_rtol"],
                               atol=g["fp32_atol"])


def test_golden_kv_len_bounds_and_progression():
    g = json.load(open(os.path.join(GOLDEN, "active_kv_progression.json")))
    cap, T = g["capacity"], g["prompt_len"]
    k, v = rnd(cap, 1, 4), rnd(cap, 1, 4)
    full_mask = np.ones((1, cap), dtype=bool)
    for kv_len in g["valid_kv_len"]:
        A.check_kv_len(kv_len, cap)
        A.attend_prefix(rnd(1, 1, 4), k, v, kv_len)
    for kv_len in g["invalid_kv_len"]:
        with pytest.raises(ValueError):
            A.check_kv_len(kv_len, cap)
        with pytest.raises(ValueError):
            A.attend_prefix(rnd(1, 1, 4), k, v, kv_len)
    lengths = []
    for kv_len in g["kv_len_probe"]:
        ks, vs, ms = A.active_slices(k, v, full_mask, kv_len)
        lengths.append([ks.shape[0], vs.shape[0], ms.shape[-1]])
    assert lengths == g["kvmask_lengths"]
    # prefill at kv_len = T, then decode step i at kv_len = T + i + 1
    progression = [T] + [T + i + 1 for i in range(2)]
    assert progression == g["kv_len_progression"]


def test_gqa_head_map_is_repeat_interleave():
    Hq, Hkv = 8, 2
    heads = torch.arange(Hkv).repeat_interleave(Hq // Hkv).tolist()
    assert [A.kv_head_of(h, Hq, Hkv) for h in range(Hq)] == heads


def test_packed_equals_padded_masked_and_per_sample():
    """TensorRT-LLM #18973: packed K/V equal the padded-and-masked result and per-sample
    runs (split-consistency, uneven boundary lengths)."""
    lens = [7, 3]
    q = rnd(2, 4, 4, 8)
    kp, vp = rnd(sum(lens), 2, 8), rnd(sum(lens), 2, 8)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, lse = A.attend_packed(q, kp, vp, cu)
    kpad = np.zeros((2, 7, 2, 8))
    vpad = np.zeros((2, 7, 2, 8))
    for b in range(2):
        kpad[b, :lens[b]] = kp[cu[b]:cu[b + 1]]
        vpad[b, :lens[b]] = vp[cu[b]:cu[b + 1]]
    for b in range(2):
        allowed = np.zeros((4, 7), dtype=bool)
        allowed[:, :lens[b]] = True
        ob = sdpa_ref(q[b], kpad[b], vpad[b], allowed)
        assert np.max(np.abs(o[b] - ob)) <= 1e-13
        os_, _ = A.attend_prefix(q[b], kp[cu[b]:cu[b + 1]], vp[cu[b]:cu[b + 1]], lens[b])
        np.testing.assert_array_equal(o[b], os_)
    for bad in ([0, 7, 7], [0, 7, 11], [1, 7, 10], [0, 11, 10]):
        with pytest.raises(ValueError):
            A.attend_packed(q, kp, vp, bad)


def test_batch_of_two_equals_two_single_runs():
    q, k, v = rnd(2, 3, 2, 8), rnd(2, 9, 2, 8), rnd(2, 9, 2, 8)
    o, lse = A.attend_batch_prefix(q, k, v, [5, 9])
    for b, kv_len in enumerate([5, 9]):
        ob, lb = A.attend_batch_prefix(q[b:b + 1], k[b:b + 1], v[b:b + 1], [kv_len])
        np.testing.assert_array_equal(o[b], ob[0])
        np.testing.assert_array_equal(lse[b], lb[0])


def test_joint_row_permutation_leaves_unmasked_attention_unchanged():
    """flashdreams #763, proposed boundary: the same permutation of key and value rows
    preserves unmasked attention."""
    q, k, v = rnd(4, 2, 8), rnd(12, 2, 8), rnd(12, 2, 8)
    perm = rng.permutation(12)
    o, lse = A.attend_prefix(q, k, v, 12)
    op, lsep = A.attend_prefix(q, k[perm], v[perm], 12)
    assert np.max(np.abs(o - op)) <= 1e-14
    assert np.max(np.abs(lse - lsep)) <= 1e-14
    # but a permutation applied to keys alone changes the result
    ok, _ = A.attend_prefix(q, k[perm], v, 12)
    assert np.max(np.abs(o - ok)) > 1e-3


def test_block_causal_degenerate_blocks():
    q, k, v = rnd(4, 2, 8), rnd(12, 2, 8), rnd(12, 2, 8)
    oc, _ = A.attend_prefix(q, k, v, 12, A.MASK_CAUSAL)
    ob1, _ = A.attend_prefix(q, k, v, 12, A.MASK_BLOCK_CAUSAL, 1)
    np.testing.assert_array_equal(oc, ob1)
    # a block that covers the whole chunk (aligned at a multiple) unmasks the chunk
    on, _ = A.attend_prefix(q, k, v, 12, A.MASK_NONE)
    ob4, _ = A.attend_prefix(q, k, v, 12, A.MASK_BLOCK_CAUSAL, 4)
    np.testing.assert_array_equal(on, ob4)


def test_flop_count():
    assert A.flops(3, 7, 4, 8, A.MASK_NONE) == 4 * 8 * 4 * 21
    assert A.flops(3, 7, 4, 8, A.MASK_CAUSAL) == 4 * 8 * 4 * (5 + 6 + 7)


# ---------------------------------------------------------------------------------------
# Planted mistakes: each plausible oracle bug must fail at least one pin above.
# ---------------------------------------------------------------------------------------

def _sdpa_pin_fails():
    try:
        for case in CASES:
            test_matches_torch_sdpa(case)
    except AssertionError:
        return True
    return False


def test_planted_wrong_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    assert _sdpa_pin_fails()


def test_planted_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(A, "default_scale", lambda D: 1.0)
    assert _sdpa_pin_fails()


def test_planted_off_by_one_causal_is_caught(monkeypatch):
    orig = A.visible_keys

    def shifted(t, Tq, kv_len, mask, block=1):
        if mask == A.MASK_CAUSAL:
            return np.arange(kv_len) < kv_len - Tq + t  # drops the diagonal
        return orig(t, Tq, kv_len, mask, block)
    monkeypatch.setattr(A, "visible_keys", shifted)
    assert _sdpa_pin_fails()


def test_planted_top_left_alignment_is_caught(monkeypatch):
    orig = A.visible_keys

    def top_left(t, Tq, kv_len, mask, block=1):
        if mask == A.MASK_CAUSAL:
            return np.arange(kv_len) <= t
        return orig(t, Tq, kv_len, mask, block)
    monkeypatch.setattr(A, "visible_keys", top_left)
    assert _sdpa_pin_fails()


def test_planted_transposed_value_operand_is_caught(monkeypatch):
    orig = A.attend_keys

    def swapped(q, k, v, allowed, scale=None):
        return orig(q, v, k, allowed, scale)  # keys and values exchanged
    monkeypatch.setattr(A, "attend_keys", swapped)
    assert _sdpa_pin_fails()
