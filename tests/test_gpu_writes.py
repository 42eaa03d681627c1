"""GPU parity of the KV-cache writes against the oracle's reference caches, bit for bit:
indexed slab writes (index and slice forms, scattered and out-of-range indices, canary
guard bands), the device cursor, and the ring over the 48-layout sweep (storage and
metadata after every reserve / write / reset)."""
import itertools

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import cache as Cc
from tests.helpers import bits_equal

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a tensor as an unsigned-integer numpy array (the oracle caches hold bits)."""
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().cpu().contiguous().view(view).numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("B,cap,n,Hkv,D", [(1, 64, 8, 2, 64), (3, 257, 37, 5, 128), (2, 96, 96, 8, 128)])
def test_indexed_write_matches_oracle(dtype, B, cap, n, Hkv, D):
    rng = np.random.default_rng(cap * 31 + n)
    guard = 16
    # canary bands before and after the cache catch any out-of-bounds write
    kbuf = torch.full((B * cap * Hkv * D + 2 * guard,), 7.0, dtype=dtype, device=DEV)
    vbuf = torch.full_like(kbuf, -3.0)
    k_cache = kbuf[guard:guard + B * cap * Hkv * D].view(B, cap, Hkv, D)
    v_cache = vbuf[guard:guard + B * cap * Hkv * D].view(B, cap, Hkv, D)
    k_cache.zero_()
    v_cache.zero_()
    ref_k = _np_bits(k_cache)
    ref_v = _np_bits(v_cache)
    for rep in range(3):
        idx = rng.permutation(cap)[:n]
        ks = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=rep, dtype={torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[dtype])
        vs = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=rep, dtype={torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[dtype])
        skv.kv_write_indexed(k_cache, v_cache, ks.to(DEV), vs.to(DEV),
                             index=torch.from_numpy(idx).to(DEV))
        ref_k, bad_k = Cc.slab_write_indexed(ref_k, _np_bits(ks), idx)
        ref_v, bad_v = Cc.slab_write_indexed(ref_v, _np_bits(vs), idx)
        assert not bad_k and not bad_v
        torch.cuda.synchronize()
        assert np.array_equal(_np_bits(k_cache), ref_k)
        assert np.array_equal(_np_bits(v_cache), ref_v)
    assert bool((kbuf[:guard] == 7).all() and (kbuf[-guard:] == 7).all())
    assert bool((vbuf[:guard] == -3).all() and (vbuf[-guard:] == -3).all())


def test_index_form_equals_slice_form_and_k_only():
    B, cap, n, Hkv, D = 2, 128, 24, 4, 128
    ks = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", dtype="bf16").to(DEV)
    vs = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", dtype="bf16").to(DEV)
    a_k = torch.zeros(B, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    a_v = torch.zeros_like(a_k)
    b_k, b_v = a_k.clone(), a_v.clone()
    c_k = a_k.clone()
    skv.kv_write_indexed(a_k, a_v, ks, vs, index=torch.arange(40, 40 + n, device=DEV))
    skv.kv_write_indexed(b_k, b_v, ks, vs, index=None, start=40)
    skv.kv_write_indexed(c_k, None, ks, None, index=None, start=40)
    torch.cuda.synchronize()
    assert bits_equal(a_k, b_k) and bits_equal(a_v, b_v) and bits_equal(a_k, c_k)
    with pytest.raises(skv.SkvError) as e:
        skv.kv_write_indexed(b_k, b_v, ks, vs, index=None, start=cap - n + 1)
    assert e.value.status == skv.SKV_ERR_RANGE


def test_out_of_range_index_skips_row_and_sets_error():
    B, cap, Hkv, D = 2, 16, 1, 64
    k_cache = torch.zeros(B, cap, Hkv, D, dtype=torch.float16, device=DEV)
    ks = torch.ones(B, 3, Hkv, D, dtype=torch.float16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.tensor([2, cap, -1], dtype=torch.int64, device=DEV)
    skv.kv_write_indexed(k_cache, None, ks, None, index=idx, err=err)
    torch.cuda.synchronize()
    ref, bad = Cc.slab_write_indexed(np.zeros((B, cap, Hkv, D)), np.ones((B, 3, Hkv, D)), [2, cap, -1])
    assert bad and int(err.item()) == skv.DEV_INDEX_RANGE
    assert np.array_equal(k_cache.double().cpu().numpy(), ref)


def test_batch_of_two_equals_two_single_writes():
    B, cap, n, Hkv, D = 2, 64, 16, 8, 128
    ks = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", dtype="bf16").to(DEV)
    idx = torch.arange(16, 32, device=DEV)
    both = torch.zeros(B, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    skv.kv_write_indexed(both, None, ks, None, index=idx)
    for b in range(B):
        one = torch.zeros(1, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
        skv.kv_write_indexed(one, None, ks[b:b + 1].contiguous(), None, index=idx)
        assert bits_equal(one[0], both[b])


def test_cursor_progression_and_overflow():
    """Device cursor: prefill of T rows then single-row steps give kv_len T, T+1, T+2
    (the fish-speech progression [3, 4, 5] for T = 3), and a step past capacity is refused."""
    cap, T = 8, 3
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(2, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    skv.kv_cursor_advance(cursor, T, cap, idx, kv_len, err)
    seen = [int(kv_len[0])]
    assert idx.tolist() == [0, 1, 2]
    one = torch.empty(1, dtype=torch.int64, device=DEV)
    for i in range(cap - T):
        skv.kv_cursor_advance(cursor, 1, cap, one, kv_len, err)
        assert one.tolist() == [T + i]
        seen.append(int(kv_len[0]))
    assert seen[:3] == [3, 4, 5] and seen[-1] == cap and int(err) == 0
    assert kv_len.tolist() == [cap, cap]
    skv.kv_cursor_advance(cursor, 1, cap, one, kv_len, err)
    assert one.tolist() == [-1] and int(err) == skv.DEV_CURSOR_FULL
    assert int(cursor) == cap and kv_len.tolist() == [cap, cap]


# ----------------------------------------------------------------------------------------
# Ring: 48 aligned layouts (sink x rolling x chunk x B), every op compared bit for bit
# ----------------------------------------------------------------------------------------
LAYOUTS = list(itertools.product([0, 1, 2], [1, 2, 3, 6], [1, 4], [1, 2]))


def _ring_ops(n_slots, rolling):
    n_first = n_slots + 2 * rolling + 1  # first eviction and two full wraps
    ops = []
    for seg, n in enumerate([n_first, 3]):
        for c in range(n):
            ops.append(("reserve", seg, c))
            for r in range(1 + c % 4):
                ops.append(("write", seg, c, r))
        if seg == 0:
            ops.append(("reserve", seg, n))  # reserved and never written, then reset
        ops.append(("reset", seg))
    return ops


@pytest.mark.parametrize("sink,rolling,C,B", LAYOUTS)
def test_ring_layout_sweep_bit_exact(sink, rolling, C, B):
    n_slots = sink + rolling
    Hkv, D = 2, 64
    k_store = torch.zeros(B, n_slots * C, Hkv, D, dtype=torch.bfloat16, device=DEV)
    v_store = torch.zeros_like(k_store)
    ring = skv.Ring(k_store, v_store, C, n_slots, sink)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sims_k = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D), dtype=np.int16) for _ in range(B)]
    sims_v = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D), dtype=np.int16) for _ in range(B)]
    compared = 0
    for op in _ring_ops(n_slots, rolling):
        if op[0] == "reserve":
            ring.reserve()
            for s in sims_k + sims_v:
                s.reserve()
        elif op[0] == "reset":
            ring.reset()
            for s in sims_k + sims_v:
                s.reset()
        else:
            _, seg, c, r = op
            chunk = 100 * seg + c
            ks = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=chunk, rewrite=r, dtype="bf16")
            vs = SI.per_batch_normal(B, (C, Hkv, D), "misc", "v", chunk=chunk, rewrite=r, dtype="bf16")
            ring.write(ks.to(DEV), vs.to(DEV), err=err)
            kb, vb = _np_bits(ks), _np_bits(vs)
            for b in range(B):
                assert sims_k[b].write(kb[b]) and sims_v[b].write(vb[b])
        torch.cuda.synchronize()
        gk, gv = _np_bits(k_store), _np_bits(v_store)
        for b in range(B):
            assert np.array_equal(gk[b], sims_k[b].storage), (op, b)
            assert np.array_equal(gv[b], sims_v[b].storage), (op, b)
            assert int(ring.kv_len[b]) == sims_k[b].valid_tokens(), (op, b)
            assert int(ring.slot[b]) == sims_k[b].current_slot(), (op, b)
            compared += 2
    assert int(err) == 0 and compared > 0


def test_ring_write_before_reserve_is_a_device_error_and_writes_nothing():
    B, C, n_slots, Hkv, D = 2, 4, 3, 1, 64
    k_store = torch.zeros(B, n_slots * C, Hkv, D, dtype=torch.float16, device=DEV)
    ring = skv.Ring(k_store, None, C, n_slots, 1)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ring.write(torch.ones(B, C, Hkv, D, dtype=torch.float16, device=DEV), err=err)
    torch.cuda.synchronize()
    assert int(err) == skv.DEV_RING_UNRESERVED and int(k_store.abs().sum()) == 0
    assert ring.kv_len.tolist() == [0, 0]


def test_ring_independent_branches_with_batch_mask():
    """Cond and uncond states advance independently (flashdreams #763, proposed boundary)."""
    B, C, n_slots, sink, Hkv, D = 2, 2, 4, 1, 1, 64
    k_store = torch.zeros(B, n_slots * C, Hkv, D, dtype=torch.bfloat16, device=DEV)
    ring = skv.Ring(k_store, None, C, n_slots, sink)
    sims = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D), dtype=np.int16) for _ in range(B)]
    only0 = torch.tensor([1, 0], dtype=torch.uint8, device=DEV)
    for step in range(9):
        mask = only0 if step % 3 else None
        active = [0] if step % 3 else [0, 1]
        ring.reserve(mask)
        src = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=step, dtype="bf16")
        ring.write(src.to(DEV), batch_mask=mask)
        bits = _np_bits(src)
        for b in active:
            sims[b].reserve()
            sims[b].write(bits[b])
        if step == 5:
            ring.reset(only0)
            sims[0].reset()
        torch.cuda.synchronize()
        g = _np_bits(k_store)
        for b in range(B):
            assert np.array_equal(g[b], sims[b].storage)
            assert int(ring.kv_len[b]) == sims[b].valid_tokens()


def test_reset_recovers_after_a_flagged_bad_write():
    """Failure recovery with the ring's own primitive: after a write the device refuses (the
    cond branch wrote without a reservation: SKV_DEV_RING_UNRESERVED, that branch untouched),
    kv_ring_reset of that branch brings it back to a state from which every further write,
    wraparound included, matches the oracle's physical ring bit for bit, and attention over
    the recovered ring matches the oracle over the same storage."""
    from oracle import attention as A
    from tests.helpers import check_attention, f64
    B, C, n_slots, sink, Hkv, Hq, D = 2, 16, 4, 1, 2, 4, 64
    k_store = torch.zeros(B, n_slots * C, Hkv, D, dtype=torch.bfloat16, device=DEV)
    v_store = torch.zeros_like(k_store)
    ring = skv.Ring(k_store, v_store, C, n_slots, sink)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sims_k = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D), dtype=np.int16) for _ in range(B)]
    sims_v = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D), dtype=np.int16) for _ in range(B)]
    only1 = torch.tensor([0, 1], dtype=torch.uint8, device=DEV)
    only0 = torch.tensor([1, 0], dtype=torch.uint8, device=DEV)

    def chunk(i):
        ks = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=60 + i, dtype="bf16")
        vs = SI.per_batch_normal(B, (C, Hkv, D), "misc", "v", chunk=60 + i, dtype="bf16")
        return ks, vs

    def step(i, mask, active):
        ring.reserve(mask)
        ks, vs = chunk(i)
        ring.write(ks.to(DEV), vs.to(DEV), batch_mask=mask, err=err)
        kb, vb = _np_bits(ks), _np_bits(vs)
        for b in active:
            sims_k[b].reserve(), sims_v[b].reserve()
            sims_k[b].write(kb[b]), sims_v[b].write(vb[b])

    def compare(what):
        torch.cuda.synchronize()
        gk, gv = _np_bits(k_store), _np_bits(v_store)
        for b in range(B):
            assert np.array_equal(gk[b], sims_k[b].storage), (what, b)
            assert np.array_equal(gv[b], sims_v[b].storage), (what, b)
            assert int(ring.kv_len[b]) == sims_k[b].valid_tokens(), (what, b)

    for i in range(3):
        step(i, None, [0, 1])
    compare("before the fault")
    # the fault: branch 0 is reset, then written with no reservation (only branch 1 reserved)
    ring.reset(only0)
    for s in (sims_k[0], sims_v[0]):
        s.reset()
    ring.reserve(only1)
    ks, vs = chunk(3)
    ring.write(ks.to(DEV), vs.to(DEV), err=err)
    for s, x in ((sims_k[1], ks), (sims_v[1], vs)):
        s.reserve()
        s.write(_np_bits(x)[1])
    compare("after the refused write")
    assert int(err) == skv.DEV_RING_UNRESERVED
    # recovery: reset the faulted branch, clear the error word, carry on past a wraparound
    err.zero_()
    ring.reset(only0)
    for s in (sims_k[0], sims_v[0]):
        s.reset()
    for i in range(4, 4 + 2 * n_slots):
        step(i, None, [0, 1])
        compare(f"recovered step {i}")
    assert int(err) == 0
    q = SI.per_batch_normal(B, (C, Hq, D), "misc", "q", chunk=99, dtype="bf16")
    o = skv.attn_chunk_fwd(q.to(DEV), k_store, v_store, kv_len_dev=ring.kv_len, max_seqlen_kv=n_slots * C)
    lens = ring.kv_len.tolist()
    def oracle_store(sim):  # the oracle's own storage (bf16 bits), not the GPU's
        return f64(torch.from_numpy(np.ascontiguousarray(sim.storage)).view(torch.bfloat16))
    refs = np.stack([A.attend_prefix(f64(q[b]), oracle_store(sims_k[b]), oracle_store(sims_v[b]), lens[b])[0]
                     for b in range(B)])
    check_attention(o, refs, "bf16", "attention over the recovered ring")
