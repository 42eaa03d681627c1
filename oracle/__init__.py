"""CPU fp64 oracle for chunk attention over a preallocated KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library (``streaming_kv_cache_write_amd``) and imports nothing from it;
callers hand it plain numpy arrays.

Sources (the four web pages this method is defined by):

* LingBot-World PR #53, "refactor(kv): index_copy_ for KV-cache writes
  (enabler for multi-user batching + CUDA Graphs)" -- indexed slab writes.
* flashdreams issue #763, "add an opt-in circular KV policy for streaming
  attention" -- the sink-plus-window ring, its reset, and the permutation
  property of unmasked attention.
* fish-speech PR #1312, "perf(text2semantic): pass only active KV cache prefix
  to SDPA" -- active-prefix attention, kv_len bounds and progression.
* TensorRT-LLM PR #18973, "FA4 variable-length cross-attention" -- K/V packed by
  cu_seqlens_kv with padded Q.

Modules:

* ``oracle.attention`` -- softmax attention written out from its definition
  (two-pass, max-subtracted, fp64), a scalar brute-force twin, the key-set
  rules (masks, active prefix, packed segments, GQA head map).
* ``oracle.cache`` -- slab writes (explicit row loop), the ring as a physical
  slot simulation that picks slots by search, a chronological history that
  defines what the ring must retain, and the chronological buffer with the
  roll-left copy that the ring replaces (the comparison arm).
* ``oracle.ragged`` -- packing of ragged K/V (each branch's valid rows
  concatenated) and its prefix-sum metadata.
* ``oracle.rope`` -- keys rotated at their absolute positions before the cache
  write (fp64 rotation, then the cache dtype's rounding), and the positions of
  ring chunks.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, brute force, library routines (torch CPU fp64 SDPA) and the values the
pages print (``tests/golden/``). Parity of the large synthetic workloads'
actual output values is pinned only through those properties; no page prints
such values.
"""
