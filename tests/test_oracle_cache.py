"""Pins of the reference caches: slab index form vs slice form vs numpy/torch
index_copy, the physical ring (slot chosen by search) vs the chronological
history definition over a 48-layout sweep, the ring's closed-form slot sequence,
and physical-prefix attention vs chronological attention."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as Cc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(777)


def test_slab_index_form_equals_slice_form_and_torch_index_copy():
    cache = rng.standard_normal((2, 16, 3, 4))
    src = rng.standard_normal((2, 5, 3, 4))
    idx = np.arange(6, 11)
    a, bad = Cc.slab_write_indexed(cache, src, idx)
    assert not bad
    b = Cc.slab_write_slice(cache, src, 6)
    np.testing.assert_array_equal(a, b)
    t = torch.from_numpy(cache.copy()).index_copy_(1, torch.from_numpy(idx), torch.from_numpy(src))
    np.testing.assert_array_equal(a, t.numpy())
    # a scattered (non-contiguous) index matches torch too
    idx2 = np.array([15, 0, 7, 3, 9])
    c, _ = Cc.slab_write_indexed(cache, src, idx2)
    t2 = torch.from_numpy(cache.copy()).index_copy_(1, torch.from_numpy(idx2), torch.from_numpy(src))
    np.testing.assert_array_equal(c, t2.numpy())


def test_slab_out_of_range_rows_are_skipped_and_flagged():
    cache = np.zeros((1, 4, 1, 2))
    src = np.ones((1, 3, 1, 2))
    out, bad = Cc.slab_write_indexed(cache, src, [1, 4, -1])
    assert bad
    expect = np.zeros((1, 4, 1, 2))
    expect[0, 1] = 1
    np.testing.assert_array_equal(out, expect)


def test_slab_batch_of_two_equals_two_single_runs():
    cache = rng.standard_normal((2, 12, 2, 4))
    for c in range(3):
        src = rng.standard_normal((2, 4, 2, 4))
        idx = np.arange(4 * c, 4 * c + 4)
        both, _ = Cc.slab_write_indexed(cache, src, idx)
        for b in range(2):
            one, _ = Cc.slab_write_indexed(cache[b:b + 1], src[b:b + 1], idx)
            np.testing.assert_array_equal(both[b], one[0])
        cache = both


def closed_form_slot(c, n_slots, sink):
    return c if c < n_slots else sink + (c - sink) % (n_slots - sink)


@pytest.mark.parametrize("n_slots,sink", [(2, 0), (2, 1), (4, 1), (7, 1), (5, 2), (3, 0)])
def test_physical_slot_choice_matches_closed_form(n_slots, sink):
    r = Cc.RingPhysical(n_slots, sink, 1, (1,))
    for c in range(3 * n_slots + 2):
        r.reserve()
        assert r.current_slot() == closed_form_slot(c, n_slots, sink)
        r.write(np.full((1, 1), float(c)))
        assert r.valid_tokens() == min(c + 1, n_slots)


def test_retained_ids_closed_form():
    h = Cc.RingChronological(7, 1)
    for c in range(12):
        h.reserve()
        h.write(np.zeros(1))
    # after chunk 11: sink 0, then the newest 6 chunks 6..11
    assert h.retained_ids() == [0, 6, 7, 8, 9, 10, 11]


def ring_sequence(n_chunks_before_reset, rewrites_of, tail_chunks):
    """Ops list: ('reserve'|'write'|'reset', chunk, rewrite)."""
    ops = []
    for seg, n in enumerate([n_chunks_before_reset, tail_chunks]):
        for c in range(n):
            ops.append(("reserve", seg, c, 0))
            for r in range(rewrites_of(c)):
                ops.append(("write", seg, c, r))
        ops.append(("reset", seg, 0, 0))
    return ops


def run_layout(sink, rolling, C, B, attend=True):
    """Drive physical and chronological rings through a sequence with repeated writes,
    a reset mid-sequence and a final reset; compare after every write. Returns the number
    of comparisons made (row-for-row logical compare + attention compare)."""
    n_slots = sink + rolling
    Hkv, D = 1, 4
    phys = [Cc.RingPhysical(n_slots, sink, C, (Hkv, D)) for _ in range(B)]
    chron = [Cc.RingChronological(n_slots, sink) for _ in range(B)]
    n_first = n_slots + 2 * rolling + 1  # first eviction and at least two wraps
    ops = ring_sequence(n_first, lambda c: 1 + (c % 4), 3)
    comparisons = 0
    for op, seg, c, r in ops:
        for b in range(B):
            if op == "reserve":
                phys[b].reserve()
                chron[b].reserve()
            elif op == "reset":
                phys[b].reset()
                chron[b].reset()
            else:
                chunk = rng.standard_normal((C, Hkv, D))
                assert phys[b].write(chunk) == chron[b].write(chunk)
                logical = phys[b].logical()
                retained = chron[b].retained()
                assert len(logical) == len(retained)
                for x, y in zip(logical, retained):
                    np.testing.assert_array_equal(x, y)
                    comparisons += 1
                assert phys[b].valid_tokens() == C * len(retained)
                if attend:
                    q = rng.standard_normal((C, 2, D))
                    kp = phys[b].physical_prefix()
                    kc = np.concatenate(retained, axis=0)
                    # values are a fixed function of each stored row, so K and V rows move
                    # together under the slot permutation
                    vp = np.tanh(kp) + 0.25
                    vc = np.tanh(kc) + 0.25
                    o1, l1 = A.attend_prefix(q, kp, vp, kp.shape[0])
                    o2, l2 = A.attend_prefix(q, kc, vc, kc.shape[0])
                    assert np.max(np.abs(o1 - o2)) <= 1e-13
                    assert np.max(np.abs(l1 - l2)) <= 1e-13
                    comparisons += 1
    return comparisons


LAYOUTS = list(itertools.product([0, 1, 2], [1, 2, 3, 6], [1, 4], [1, 2]))


def test_layout_count_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "ring_prototype.json")))
    assert len(LAYOUTS) == g["aligned_layouts"]


@pytest.mark.parametrize("sink,rolling,C,B", LAYOUTS)
def test_ring_physical_equals_chronological(sink, rolling, C, B):
    assert run_layout(sink, rolling, C, B) > 0


def test_write_without_reserve_is_rejected_and_reset_keeps_stale_rows():
    r = Cc.RingPhysical(3, 1, 2, (1,))
    assert not r.write(np.ones((2, 1)))
    r.reserve()
    assert r.write(np.full((2, 1), 5.0))
    r.reset()
    assert r.valid_tokens() == 0
    assert not r.write(np.ones((2, 1)))
    np.testing.assert_array_equal(r.storage[:2], 5.0)  # stale rows stay


def test_reserve_is_idempotent_until_written():
    r = Cc.RingPhysical(3, 1, 1, (1,))
    h = Cc.RingChronological(3, 1)
    for ring in (r, h):
        ring.reserve()
        ring.reserve()
        ring.write(np.ones((1, 1)))
    assert r.valid_tokens() == 1 and h.retained_ids() == [0]


def test_planted_wrong_eviction_is_caught(monkeypatch):
    """Evicting the newest non-sink chunk instead of the oldest must fail the sweep."""
    def newest(self):
        empty = [s for s in range(self.n_slots) if self.slot_chunk[s] is None]
        if empty:
            return min(empty)
        return max((cid, s) for s, cid in enumerate(self.slot_chunk) if cid >= self.sink)[1]
    monkeypatch.setattr(Cc.RingPhysical, "_choose_slot", newest)
    with pytest.raises(AssertionError):
        run_layout(1, 3, 2, 1, attend=False)


def test_planted_unpinned_sink_is_caught(monkeypatch):
    def no_sink(self):
        empty = [s for s in range(self.n_slots) if self.slot_chunk[s] is None]
        if empty:
            return min(empty)
        return min((cid, s) for s, cid in enumerate(self.slot_chunk))[1]
    monkeypatch.setattr(Cc.RingPhysical, "_choose_slot", no_sink)
    with pytest.raises(AssertionError):
        run_layout(1, 3, 2, 1, attend=False)


# ----------------------------------------------------------------------------------------
# The chronological roll-left buffer (comparison arm), pinned to the chunk history
# ----------------------------------------------------------------------------------------

def run_rolling(sink, rolling, C, B):
    """Drive the roll-left buffer and the chronological history through the same sequence
    (repeated writes, a reset mid-sequence); compare the buffer's valid rows with the
    retained chunks after every write. Returns the number of comparisons."""
    n_slots = sink + rolling
    Hkv, D = 1, 3
    roll = [Cc.RollingChronological(n_slots, sink, C, (Hkv, D)) for _ in range(B)]
    chron = [Cc.RingChronological(n_slots, sink) for _ in range(B)]
    ops = ring_sequence(n_slots + 2 * rolling + 1, lambda c: 1 + (c % 3), 3)
    n = 0
    for op, seg, c, r in ops:
        for b in range(B):
            if op == "reserve":
                roll[b].reserve()
                chron[b].reserve()
            elif op == "reset":
                roll[b].reset()
                chron[b].reset()
            else:
                chunk = rng.standard_normal((C, Hkv, D))
                assert roll[b].write(chunk) == chron[b].write(chunk)
                np.testing.assert_array_equal(roll[b].valid(), np.concatenate(chron[b].retained(), axis=0))
                n += 1
    return n


@pytest.mark.parametrize("sink,rolling,C,B", LAYOUTS)
def test_rolling_buffer_equals_chronological(sink, rolling, C, B):
    assert run_rolling(sink, rolling, C, B) > 0


def test_roll_left_fixture():
    """Rows labelled by position: sink 2 rows, shift 3, 10 rows -> rows 5..9 move to 2..6,
    rows 0, 1 stay, rows 7..9 keep their old contents."""
    x = np.arange(10, dtype=np.float64)[:, None]
    y = Cc.roll_left(x, 2, 3, 10)
    np.testing.assert_array_equal(y[:, 0], [0, 1, 5, 6, 7, 8, 9, 7, 8, 9])
    with pytest.raises(ValueError):
        Cc.roll_left(x, 8, 3, 10)


def test_rolling_counts_one_roll_per_new_chunk_once_full():
    """7 slots, sink 1, 12 chunks with 4 writes each: rolls start at chunk 7 (the first that
    does not fit) -> 5 rolls, 23400 rows moved per roll for C = 4680 (the f2 figure)."""
    r = Cc.RollingChronological(7, 1, 2, (1,))
    for c in range(12):
        r.reserve()
        for _ in range(4):
            r.write(np.full((2, 1), float(c)))
    assert r.rolls == 5
    np.testing.assert_array_equal(r.valid()[:, 0], [0, 0, 6, 6, 7, 7, 8, 8, 9, 9, 10, 10, 11, 11])
    assert (7 - 1 - 1) * 4680 == 23400


def test_planted_roll_without_sink_is_caught(monkeypatch):
    real = Cc.roll_left
    monkeypatch.setattr(Cc, "roll_left", lambda s, sink, shift, rows: real(s, 0, shift, rows))
    with pytest.raises(AssertionError):
        run_rolling(1, 3, 2, 1)
