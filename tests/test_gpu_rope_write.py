"""Writes with keys rotated at their absolute positions (kv_write_indexed_rope,
kv_ring_write_rope) against the fp64 oracle (oracle.rope): cache contents bit-exact for bf16
and fp16 (fp32: within one ulp, the only freedom being the last bit of the fp64 sine and
cosine), V copied unchanged, rows outside the write untouched, out-of-range indices skipped and
reported; the ring's rotation follows chunk chronology through rewrites, wraparound, a reset
and a per-element mask; and prefix attention over the ring equals attention over the
chronological history of rotated keys."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from oracle import cache as Cc
from oracle import rope as R
from tests.helpers import check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def inv_freq(D, base=10000.0):
    return base ** (-np.arange(D // 2) * 2.0 / D)


def assert_cache_equal(got: torch.Tensor, want: np.ndarray, dtype: str, what: str):
    g = f64(got)
    if dtype == "f32":
        ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        bad = np.abs(g - want) > ulp
        assert not bad.any(), f"{what}: {int(bad.sum())} values off by more than one ulp"
    else:
        same = (g == want) | (np.isnan(g) & np.isnan(want))
        assert same.all(), f"{what}: {int((~same).sum())} of {same.size} values differ"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("layout", [skv.ROPE_HALF, skv.ROPE_INTERLEAVED])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["index", "slice"])
def test_indexed_rope_write_matches_oracle(dtype, layout, D, mode):
    B, cap, n, Hkv = 2, 300, 37, 3
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=51, dtype=dtype)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=51, dtype=dtype)
    fill = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "q", chunk=52, dtype=dtype)  # canary rows
    kc, vc = fill.clone().to(DEV), fill.clone().to(DEV)
    f = inv_freq(D)
    if mode == "index":
        rows = np.random.default_rng(7).permutation(cap)[:n].astype(np.int64)
        idx = torch.from_numpy(rows).to(DEV)
        start = 0
    else:
        rows = np.arange(250, 250 + n, dtype=np.int64)
        idx, start = None, 250
    skv.kv_write_indexed_rope(kc, vc, k.to(DEV), v.to(DEV), torch.from_numpy(f).to(DEV),
                              rope_layout=layout, index=idx, start=start)
    want_k, want_v = f64(fill), f64(fill)
    for b in range(B):
        want_k[b, rows] = R.rope_keys(f64(k[b]), rows, f, layout, dtype)
        want_v[b, rows] = f64(v[b])
    assert_cache_equal(kc, want_k, dtype, "K cache")
    assert_cache_equal(vc, want_v, dtype, "V cache")


def test_indexed_rope_large_positions_and_bad_index():
    dtype, D, Hkv, n, cap = "bf16", 128, 2, 20, 60000
    k = SI.per_batch_normal(1, (n, Hkv, D), "misc", "k", chunk=53, dtype=dtype)
    kc = torch.zeros(1, cap, Hkv, D, dtype=TD[dtype], device=DEV)
    rows = np.array(list(range(59980, 59999)) + [cap + 5], dtype=np.int64)  # last one out of range
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    f = inv_freq(D, base=500000.0)
    skv.kv_write_indexed_rope(kc, None, k.to(DEV), None, torch.from_numpy(f).to(DEV),
                              index=torch.from_numpy(rows).to(DEV), err=err)
    assert int(err.item()) & skv.DEV_INDEX_RANGE
    want = np.zeros((cap, Hkv, D))
    want[rows[:-1]] = R.rope_keys(f64(k[0, :-1]), rows[:-1], f, R.LAYOUT_HALF, dtype)
    assert_cache_equal(kc[0, 59900:], want[59900:], dtype, "K cache tail")
    assert not kc[0, :59900].any()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("layout", [skv.ROPE_HALF, skv.ROPE_INTERLEAVED])
def test_ring_rope_lifecycle(dtype, layout):
    """Every write, rewrite, wrap and reset against oracle rings (one per batch element) whose
    chunks are rotated at chunk_id * C + t."""
    B, C, n_slots, sink, Hkv, D = 2, 37, 4, 1, 2, 128
    ks = torch.zeros(B, n_slots * C, Hkv, D, dtype=TD[dtype], device=DEV)
    vs = torch.zeros_like(ks)
    ring = skv.Ring(ks, vs, C, n_slots, sink)
    f = inv_freq(D)
    fd = torch.from_numpy(f).to(DEV)
    ok_k = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D)) for _ in range(B)]
    ok_v = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D)) for _ in range(B)]
    chunk_id = [0] * B  # id of the chunk each element's next reservation gets
    cur = [None] * B
    only1 = torch.tensor([0, 1], dtype=torch.uint8, device=DEV)
    # (action, mask): reserve+2 rewrites per chunk; a reset after chunk 6; element 1 alone later
    plan = [("chunk", None)] * 7 + [("reset", None)] + [("chunk", None)] * 2 + [("chunk", "only1")]
    step = 0
    for action, m in plan:
        sel = [True, True] if m is None else [False, True]
        bm = None if m is None else only1
        if action == "reset":
            ring.reset(bm)
            for b in range(B):
                if sel[b]:
                    ok_k[b].reset(); ok_v[b].reset(); chunk_id[b] = 0
            continue
        ring.reserve(bm)
        for b in range(B):
            if sel[b]:
                ok_k[b].reserve(); ok_v[b].reserve()
                cur[b] = chunk_id[b]; chunk_id[b] += 1
        for rewrite in range(2):
            step += 1
            k = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=60 + step, dtype=dtype)
            v = SI.per_batch_normal(B, (C, Hkv, D), "misc", "v", chunk=60 + step, dtype=dtype)
            ring.write_rope(k.to(DEV), v.to(DEV), fd, rope_layout=layout, batch_mask=bm)
            for b in range(B):
                if sel[b]:
                    ok_k[b].write(R.rope_keys(f64(k[b]), R.ring_positions(cur[b], C), f, layout, dtype))
                    ok_v[b].write(f64(v[b]))
            for b in range(B):
                assert_cache_equal(ks[b], ok_k[b].storage, dtype, f"K step {step} b {b}")
                assert_cache_equal(vs[b], ok_v[b].storage, dtype, f"V step {step} b {b}")
                assert int(ring.kv_len[b].item()) == ok_k[b].valid_tokens()
    ring.close()


def test_ring_rope_attention_equals_chronological_history():
    """The point of rotating before storage: unmasked prefix attention over the ring's
    physical rows equals attention over the retained chunks in time order."""
    dtype, B, C, n_slots, sink, Hq, Hkv, D = "bf16", 1, 64, 4, 1, 4, 2, 128
    ks = torch.zeros(B, n_slots * C, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vs = torch.zeros_like(ks)
    ring = skv.Ring(ks, vs, C, n_slots, sink)
    f = inv_freq(D)
    fd = torch.from_numpy(f).to(DEV)
    hist_k, hist_v = Cc.RingChronological(n_slots, sink), Cc.RingChronological(n_slots, sink)
    for cid in range(6):
        k = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=80 + cid, dtype=dtype)
        v = SI.per_batch_normal(B, (C, Hkv, D), "misc", "v", chunk=80 + cid, dtype=dtype)
        ring.reserve()
        ring.write_rope(k.to(DEV), v.to(DEV), fd)
        hist_k.reserve(); hist_v.reserve()
        hist_k.write(R.rope_keys(f64(k[0]), R.ring_positions(cid, C), f, R.LAYOUT_HALF, dtype))
        hist_v.write(f64(v[0]))
    q = SI.per_batch_normal(B, (C, Hq, D), "misc", "q", chunk=90, dtype=dtype)
    o = skv.attn_chunk_fwd(q.to(DEV), ks, vs, kv_len_dev=ring.kv_len, max_seqlen_kv=n_slots * C)
    kchron = np.concatenate(hist_k.retained())
    vchron = np.concatenate(hist_v.retained())
    ref, _ = A.attend_prefix(f64(q[0]), kchron, vchron, len(kchron), A.MASK_NONE)
    check_attention(o[0], ref, dtype, "ring with rotated keys")
    ring.close()


@pytest.mark.parametrize("shape", [
    (16, 1, 1000),    # D=16, one head: 256 tokens per workgroup, the angle table exactly full
    (512, 5, 37),     # 160 units per token, 6 tokens per workgroup
    (1024, 17, 9),    # 1088 units per token: one token per workgroup, two passes of 1024 units
    (64, 3, 1),       # a single token
])
@pytest.mark.parametrize("layout", [skv.ROPE_HALF, skv.ROPE_INTERLEAVED])
def test_indexed_rope_write_block_shapes(shape, layout):
    """Token blocks of every size the kernel plans: many tokens per workgroup with a full angle
    table, a few, and one token whose units take two passes."""
    D, Hkv, n = shape
    dtype, B, cap = "bf16", 2, n + 50
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=70 + D, dtype=dtype)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=70 + D, dtype=dtype)
    kc = torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV)
    vc = torch.zeros_like(kc)
    rows = np.random.default_rng(D + n).permutation(cap)[:n].astype(np.int64)
    f = inv_freq(D)
    skv.kv_write_indexed_rope(kc, vc, k.to(DEV), v.to(DEV), torch.from_numpy(f).to(DEV),
                              rope_layout=layout, index=torch.from_numpy(rows).to(DEV))
    want_k, want_v = np.zeros((B, cap, Hkv, D)), np.zeros((B, cap, Hkv, D))
    for b in range(B):
        want_k[b, rows] = R.rope_keys(f64(k[b]), rows, f, layout, dtype)
        want_v[b, rows] = f64(v[b])
    assert_cache_equal(kc, want_k, dtype, f"K cache {shape}")
    assert_cache_equal(vc, want_v, dtype, f"V cache {shape}")
