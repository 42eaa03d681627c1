"""Reference KV caches: indexed slab writes and the sink-plus-window ring.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): product code never
imports this module.

Slab (LingBot-World PR #53 "refactor(kv): index_copy_ for KV-cache writes
(enabler for multi-user batching + CUDA Graphs)", section Summary): a per-user
cache [B, cap, Hkv, D] with the sequence on dim 1; a chunk of n rows is written
with index_copy along dim 1 at a length-n index vector that every batch element
shares (section What this is and isn't: homogeneous batching). With a
contiguous index it must equal the slice assignment cache[:, s:s+n] = src
(section Summary and Verification).

Ring (flashdreams issue #763 "add an opt-in circular KV policy for streaming
attention", sections current path and proposed boundary): storage of n_slots
whole chunks of C tokens per batch element; the first S chunks since the last
reset are a pinned sink, the remaining slots hold the newest chunks. A chunk's
slot is reserved separately from its writes, so the repeated denoising writes
of one chunk all land in the same slot. Reset forgets the contents. Cond and
uncond branches keep independent state.

Three independent formulations are kept, and the tests pin them to each other:

* ``RingChronological`` -- the history of chunks since reset, in order; the
  retained set is the sink chunks followed by the newest chunks that fit.
* ``RingPhysical`` -- slot-by-slot storage. A new chunk takes the lowest empty
  slot, else the slot holding the oldest non-sink chunk, found by searching
  the slots' chunk ids (no closed-form slot formula). Reset empties every slot
  but leaves the stale rows in place.
* ``RollingChronological`` -- the chronological buffer the page's current path
  keeps (section current path: when a new chunk overflows the window, the
  retained window is copied left by one chunk): rows in time order, the sink
  chunks first, a full buffer moved left past the sink by one chunk (``roll_left``)
  before the new chunk goes to its end.

Readings taken where the page is silent:

* reserve while the previous reservation is still unwritten keeps that
  reservation (it is idempotent until a write happens);
* the retained token count grows at the first write after a reserve, so
  attention between reserve and write sees the previous retained set;
* a write with no reservation since the last reset writes nothing and
  reports an error.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------------------
# Slab
# ----------------------------------------------------------------------------------------

def slab_write_indexed(cache: np.ndarray, src: np.ndarray, index) -> tuple[np.ndarray, bool]:
    """index_copy along the sequence dim, written as an explicit row loop:
    cache[b, index[t]] = src[b, t] for every b and t.

    cache [B, cap, ...], src [B, n, ...], index [n] (one vector shared by all B).
    Rows whose index is outside [0, cap) are skipped and flagged, mirroring the
    library's device error word. Returns (new cache, any_out_of_range).
    """
    out = cache.copy()
    B, cap = cache.shape[:2]
    index = [int(i) for i in index]
    if src.shape[0] != B or src.shape[1] != len(index) or src.shape[2:] != cache.shape[2:]:
        raise ValueError("src shape does not match cache / index")
    bad = False
    for b in range(B):
        for t, row in enumerate(index):
            if 0 <= row < cap:
                out[b, row] = src[b, t]
            else:
                bad = True
    return out, bad


def slab_write_slice(cache: np.ndarray, src: np.ndarray, start: int) -> np.ndarray:
    """The slice-assignment form cache[:, start:start+n] = src."""
    out = cache.copy()
    n = src.shape[1]
    if start < 0 or start + n > cache.shape[1]:
        raise ValueError("slice outside the cache")
    out[:, start:start + n] = src
    return out


# ----------------------------------------------------------------------------------------
# Ring: chronological definition
# ----------------------------------------------------------------------------------------

class RingChronological:
    """What a sink-plus-window cache must retain, defined on the chunk history alone.

    history[i] is chunk i since the last reset (its latest write). With S sink
    chunks and n_slots chunks of storage, the retained chunks after chunk c
    (0-based) are 0..S-1 followed by max(S, c+1-(n_slots-S)) .. c.
    """

    def __init__(self, n_slots: int, sink: int):
        if not (0 <= sink < n_slots):
            raise ValueError("need 0 <= sink < n_slots")
        self.n_slots, self.sink = n_slots, sink
        self.history: list[np.ndarray] = []
        self.open = False  # a reserved chunk awaits its first write

    def reserve(self) -> None:
        self.open = True

    def write(self, chunk: np.ndarray) -> bool:
        """Store the latest contents of the current chunk. Returns False (and stores
        nothing) when no chunk was ever reserved since reset."""
        if self.open:
            self.history.append(chunk.copy())
            self.open = False
            return True
        if not self.history:
            return False
        self.history[-1] = chunk.copy()
        return True

    def reset(self) -> None:
        self.history = []
        self.open = False

    def retained_ids(self) -> list[int]:
        c = len(self.history) - 1
        if c < 0:
            return []
        sink_ids = list(range(min(self.sink, c + 1)))
        window_start = max(self.sink, c + 1 - (self.n_slots - self.sink))
        return sink_ids + list(range(window_start, c + 1))

    def retained(self) -> list[np.ndarray]:
        """Retained chunk contents, oldest to newest."""
        return [self.history[i] for i in self.retained_ids()]


# ----------------------------------------------------------------------------------------
# Ring: physical slot simulation
# ----------------------------------------------------------------------------------------

class RingPhysical:
    """Slot storage [n_slots * C, ...] for one batch element, slot choice by search."""

    def __init__(self, n_slots: int, sink: int, C: int, row_shape: tuple, dtype=np.float64,
                 storage: np.ndarray | None = None):
        if not (0 <= sink < n_slots):
            raise ValueError("need 0 <= sink < n_slots")
        self.n_slots, self.sink, self.C = n_slots, sink, C
        self.storage = (np.zeros((n_slots * C,) + tuple(row_shape), dtype=dtype)
                        if storage is None else storage.copy())
        self.slot_chunk: list[int | None] = [None] * n_slots  # chunk id held by each slot
        self.next_id = 0          # id the next reserved chunk gets
        self.target: int | None = None  # slot of the current chunk
        self.pending = False      # reserved, not yet written

    def _choose_slot(self) -> int:
        empty = [s for s in range(self.n_slots) if self.slot_chunk[s] is None]
        if empty:
            return min(empty)
        # every slot is full: evict the oldest chunk that is not one of the first `sink`
        candidates = [(cid, s) for s, cid in enumerate(self.slot_chunk) if cid >= self.sink]
        return min(candidates)[1]

    def reserve(self) -> None:
        if self.pending:
            return  # still unwritten: keep the same reservation
        self.target = self._choose_slot()
        self.pending = True

    def write(self, chunk: np.ndarray) -> bool:
        if self.target is None:
            return False
        s = self.target
        self.storage[s * self.C:(s + 1) * self.C] = chunk
        if self.pending:
            self.slot_chunk[s] = self.next_id
            self.next_id += 1
            self.pending = False
        return True

    def reset(self) -> None:
        self.slot_chunk = [None] * self.n_slots
        self.next_id = 0
        self.target = None
        self.pending = False

    def valid_tokens(self) -> int:
        """Tokens attention may read: the occupied slots, which must be a physical prefix."""
        occupied = [s for s in range(self.n_slots) if self.slot_chunk[s] is not None]
        if occupied != list(range(len(occupied))):
            raise AssertionError(f"occupied slots {occupied} are not a physical prefix")
        return len(occupied) * self.C

    def current_slot(self) -> int:
        return -1 if self.target is None else self.target

    def logical(self) -> list[np.ndarray]:
        """Occupied slots' contents ordered by chunk id (oldest first)."""
        pairs = sorted((cid, s) for s, cid in enumerate(self.slot_chunk) if cid is not None)
        return [self.storage[s * self.C:(s + 1) * self.C] for _, s in pairs]

    def physical_prefix(self) -> np.ndarray:
        """Rows [0, valid_tokens) in physical slot order: what prefix attention reads."""
        return self.storage[:self.valid_tokens()]


# ----------------------------------------------------------------------------------------
# Chronological buffer with roll-left (the comparison arm)
# ----------------------------------------------------------------------------------------

def roll_left(store: np.ndarray, sink_rows: int, shift_rows: int, rows: int) -> np.ndarray:
    """Move rows [sink_rows + shift_rows, rows) of store to [sink_rows, rows - shift_rows);
    rows outside [sink_rows, rows - shift_rows) keep their contents (flashdreams issue #763,
    section current path: the retained tokens are copied left by one chunk). Defined as a
    copy of the moved block, so an overlap of source and destination does not matter."""
    if not (0 <= sink_rows and 0 < shift_rows and sink_rows + shift_rows <= rows <= store.shape[0]):
        raise ValueError(f"bad roll: sink {sink_rows}, shift {shift_rows}, rows {rows}")
    out = store.copy()
    out[sink_rows:rows - shift_rows] = store[sink_rows + shift_rows:rows].copy()
    return out


class RollingChronological:
    """Chronological buffer of n_slots * C rows for one batch element, as the page's current
    path keeps it. The chunk lifecycle matches the ring's (reserve, then one or more writes of
    the same chunk, reset); only the placement differs: a chunk goes to the end of the filled
    rows, and when the buffer is full the non-sink part first moves left by one chunk."""

    def __init__(self, n_slots: int, sink: int, C: int, row_shape: tuple, dtype=np.float64):
        if not (0 <= sink < n_slots):
            raise ValueError("need 0 <= sink < n_slots")
        self.n_slots, self.sink, self.C = n_slots, sink, C
        self.rows = n_slots * C
        self.store = np.zeros((self.rows,) + tuple(row_shape), dtype=dtype)
        self.filled = 0       # rows holding retained tokens, a multiple of C
        self.chunks = 0       # chunks since reset
        self.open = False     # a reserved chunk awaits its first write
        self.rolls = 0        # roll_left calls so far (the maintenance the ring avoids)

    def reserve(self) -> None:
        self.open = True

    def write(self, chunk: np.ndarray) -> bool:
        """First write after a reserve places a new chunk (rolling if full); later writes
        replace the current chunk. Returns False when nothing was ever reserved since reset."""
        if self.open:
            if self.filled + self.C > self.rows:  # full: drop the oldest non-sink chunk
                self.store = roll_left(self.store, self.sink * self.C, self.C, self.rows)
                self.rolls += 1
            else:
                self.filled += self.C
            self.chunks += 1
            self.open = False
        elif self.chunks == 0:
            return False
        self.store[self.filled - self.C:self.filled] = chunk
        return True

    def reset(self) -> None:
        self.filled = 0
        self.chunks = 0
        self.open = False

    def valid(self) -> np.ndarray:
        """The retained rows, oldest to newest."""
        return self.store[:self.filled]
