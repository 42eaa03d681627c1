"""HIP-graph capture and replay of the write + attention lifecycle.

The write position, ring slot and active prefix live in device memory, so a recorded
sequence keeps advancing on replay instead of rewriting the slot it saw at capture time
(flashdreams issue #763, proposed boundary; LingBot-World PR #53, What this is and isn't).
Each test replays a graph several times with eager work and synchronizations in between and
checks every replay: bit-identical to the eager run, and cache/ring state equal to the
oracle's."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from oracle import cache as Cc
from tests.helpers import bits_equal, check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm run on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_loop_graph_replays_match_eager_and_oracle():
    Hq, Hkv, D, cap, T, steps = 8, 2, 128, 512, 37, 40
    n = T + steps
    q = SI.per_batch_normal(1, (n, Hq, D), "misc", "q", chunk=501, dtype="bf16").to(DEV)
    k = SI.per_batch_normal(1, (n, Hkv, D), "misc", "k", chunk=501, dtype="bf16").to(DEV)
    v = SI.per_batch_normal(1, (n, Hkv, D), "misc", "v", chunk=501, dtype="bf16").to(DEV)
    kc = torch.zeros(1, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx_pre = torch.empty(T, dtype=torch.int64, device=DEV)
    idx = torch.empty(1, dtype=torch.int64, device=DEV)
    out_pre = torch.empty(1, T, Hq, D, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(steps, 1, 1, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(skv.attn_workspace_bytes(q[:, :1], kc, kv_len_dev=kv_len, max_seqlen_kv=n),
                     dtype=torch.uint8, device=DEV)

    def job():
        cursor.zero_()
        kc.zero_()
        vc.zero_()
        skv.kv_cursor_advance(cursor, T, cap, idx_pre, kv_len)
        skv.kv_write_indexed(kc, vc, k[:, :T], v[:, :T], index=idx_pre)
        skv.attn_chunk_fwd(q[:, :T], kc, vc, out_pre, kv_len_dev=kv_len, mask=skv.MASK_CAUSAL,
                           max_seqlen_kv=n)
        for i in range(steps):
            skv.kv_cursor_advance(cursor, 1, cap, idx, kv_len)
            skv.kv_write_indexed(kc, vc, k[:, T + i:T + i + 1], v[:, T + i:T + i + 1], index=idx)
            skv.attn_chunk_fwd(q[:, T + i:T + i + 1], kc, vc, out[i], kv_len_dev=kv_len,
                               max_seqlen_kv=n, workspace=ws)

    job()
    torch.cuda.synchronize()
    eager_out, eager_pre, eager_k = out.clone(), out_pre.clone(), kc.clone()
    g = _capture(job)
    for rep in range(3):
        out.fill_(7.0)
        out_pre.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(out, eager_out), rep
        assert bits_equal(out_pre, eager_pre), rep
        assert bits_equal(kc, eager_k), rep
        assert int(cursor) == n and int(kv_len) == n
        # eager work between replays
        skv.attn_chunk_fwd(q[:, :1], kc, vc, kv_len=5)
        torch.cuda.synchronize()
    kf, vf, qf = f64(k[0]), f64(v[0]), f64(q[0])
    refs = np.stack([A.attend_prefix(qf[T + i:T + i + 1], kf, vf, T + i + 1)[0][0] for i in range(steps)])
    check_attention(out[:, 0, 0], refs, "bf16", "graph decode")


def test_ring_chunk_step_graph_advances_slot_on_every_replay():
    """One recorded chunk step (reserve + 4 x (write + attention)) replayed for successive
    chunks: every replay lands in the next slot of the sink-plus-window schedule."""
    B, C, n_slots, sink, H, D, rewrites = 2, 64, 4, 1, 2, 128, 4
    rows = n_slots * C
    ks = torch.zeros(B, rows, H, D, dtype=torch.bfloat16, device=DEV)
    vs = torch.zeros_like(ks)
    ring = skv.Ring(ks, vs, C, n_slots, sink)
    # staging buffers the recorded step reads; the host refills them before each replay
    k_in = torch.empty(rewrites, B, C, H, D, dtype=torch.bfloat16, device=DEV)
    v_in = torch.empty_like(k_in)
    q_in = torch.empty_like(k_in)
    out = torch.empty(rewrites, B, C, H, D, dtype=torch.bfloat16, device=DEV)

    def chunk_step():
        ring.reserve()
        for r in range(rewrites):
            ring.write(k_in[r], v_in[r])
            skv.attn_chunk_fwd(q_in[r], ks, vs, out[r], kv_len_dev=ring.kv_len, max_seqlen_kv=rows)

    def fill(c):
        for r in range(rewrites):
            q_in[r].copy_(SI.per_batch_normal(B, (C, H, D), "misc", "q", chunk=900 + c, rewrite=r, dtype="bf16"))
            k_in[r].copy_(SI.per_batch_normal(B, (C, H, D), "misc", "k", chunk=900 + c, rewrite=r, dtype="bf16"))
            v_in[r].copy_(SI.per_batch_normal(B, (C, H, D), "misc", "v", chunk=900 + c, rewrite=r, dtype="bf16"))

    fill(0)
    g = _capture(chunk_step)  # the warm-up run advanced the ring eagerly: start over
    ring.reset()
    torch.cuda.synchronize()
    sims_k = [Cc.RingPhysical(n_slots, sink, C, (H, D)) for _ in range(B)]
    sims_v = [Cc.RingPhysical(n_slots, sink, C, (H, D)) for _ in range(B)]
    for c in range(2 * n_slots + 1):  # first eviction and a wrap
        fill(c)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in sims_k + sims_v:
            s.reserve()
        for r in range(rewrites):
            for b in range(B):
                sims_k[b].write(f64(k_in[r, b]))
                sims_v[b].write(f64(v_in[r, b]))
        assert ring.slot.tolist() == [s.current_slot() for s in sims_k], c
        assert ring.kv_len.tolist() == [s.valid_tokens() for s in sims_k], c
        for b in range(B):
            assert np.array_equal(f64(ks[b]), sims_k[b].storage), (c, b)
            assert np.array_equal(f64(vs[b]), sims_v[b].storage), (c, b)
            L = sims_k[b].valid_tokens()
            ref, _ = A.attend_prefix(f64(q_in[-1, b]), sims_k[b].storage[:L], sims_v[b].storage[:L], L)
            check_attention(out[-1, b], ref, "bf16", f"chunk {c} b{b}")
        skv.attn_chunk_fwd(q_in[0], ks, vs, kv_len=C)  # eager work between replays
        torch.cuda.synchronize()
