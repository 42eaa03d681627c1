"""The fused single-launch decode step (attn_decode_step) against the three-call sequence
kv_cursor_advance + kv_write_indexed + attn_chunk_fwd(kv_len_dev) and against the oracle:
outputs and caches bit-identical, cursor and kv_len progression as in the fish-speech
regression tests (prefill at T, decode step i at T+i+1), overflow refused on the device, and
graph replay."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import bits_equal, check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,Tq,Hq,Hkv,D,mask", [
    (1, 1, 32, 8, 128, 0),   # the decode workload's heads
    (2, 2, 8, 2, 128, 1),    # two-token causal steps, GQA 4:1
    (3, 1, 4, 4, 64, 0),
    (1, 4, 4, 1, 128, 1),    # 16 query rows per KV head
])
def test_fused_step_equals_three_calls(dtype, B, Tq, Hq, Hkv, D, mask):
    cap, T, steps = 300, 45, 24
    n = T + steps * Tq
    q = SI.per_batch_normal(B, (n, Hq, D), "misc", "q", chunk=31, dtype=dtype).to(DEV)
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=31, dtype=dtype).to(DEV)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=31, dtype=dtype).to(DEV)
    caches = [(torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV),
               torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV)) for _ in range(2)]
    cursors = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2)]
    lens = [torch.zeros(B, dtype=torch.int32, device=DEV) for _ in range(2)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    for (kc, vc), cur, kl in zip(caches, cursors, lens):  # shared prefill
        skv.kv_cursor_advance(cur, T, cap, idx, kl)
        skv.kv_write_indexed(kc, vc, k[:, :T].contiguous(), v[:, :T].contiguous(), index=idx)
    ws = torch.zeros(skv.attn_workspace_bytes(q[:, :Tq].contiguous(), caches[0][0], kv_len=cap,
                                              mask=mask), dtype=torch.uint8, device=DEV)
    one = torch.empty(Tq, dtype=torch.int64, device=DEV)
    kf, vf, qf = f64(k), f64(v), f64(q)
    got, want = [], []
    for i in range(steps):
        s = T + i * Tq
        qs, ks, vs = (x[:, s:s + Tq].contiguous() for x in (q, k, v))
        fused = skv.attn_decode_step(qs, ks, vs, caches[0][0], caches[0][1], cursors[0],
                                     kv_len_out=lens[0], mask=mask, workspace=ws, err=err)
        skv.kv_cursor_advance(cursors[1], Tq, cap, one, lens[1])
        skv.kv_write_indexed(caches[1][0], caches[1][1], ks, vs, index=one)
        three = skv.attn_chunk_fwd(qs, caches[1][0], caches[1][1], kv_len_dev=lens[1], mask=mask,
                                   max_seqlen_kv=cap)
        assert bits_equal(fused, three), i
        for b in range(B):
            ref, _ = A.attend_prefix(qf[b, s:s + Tq], kf[b], vf[b], s + Tq, mask)
            got.append(f64(fused[b]))
            want.append(ref)
    torch.cuda.synchronize()
    assert int(err) == 0
    assert bits_equal(caches[0][0], caches[1][0]) and bits_equal(caches[0][1], caches[1][1])
    assert int(cursors[0]) == n and lens[0].tolist() == [n] * B
    check_attention(np.stack(got), np.stack(want), dtype, "fused decode steps")


def test_fused_step_progression_and_overflow():
    """cap 8, prompt 3: the step lengths run 4, 5, ..., 8 (fish-speech #1312 progression
    [3, 4, 5] and the maximum valid prefix 8); a ninth row is refused on the device."""
    B, Hq, Hkv, D, cap, T = 1, 4, 2, 128, 8, 3
    q = SI.per_batch_normal(B, (cap + 1, Hq, D), "misc", "q", chunk=5, dtype="bf16").to(DEV)
    k = SI.per_batch_normal(B, (cap + 1, Hkv, D), "misc", "k", chunk=5, dtype="bf16").to(DEV)
    v = SI.per_batch_normal(B, (cap + 1, Hkv, D), "misc", "v", chunk=5, dtype="bf16").to(DEV)
    kc = torch.zeros(B, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(B, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    skv.kv_cursor_advance(cursor, T, cap, idx, kv_len)
    skv.kv_write_indexed(kc, vc, k[:, :T].contiguous(), v[:, :T].contiguous(), index=idx)
    seen = [int(kv_len[0])]
    for i in range(cap - T):
        o = skv.attn_decode_step(q[:, T + i:T + i + 1].contiguous(), k[:, T + i:T + i + 1].contiguous(),
                                 v[:, T + i:T + i + 1].contiguous(), kc, vc, cursor, kv_len_out=kv_len,
                                 err=err)
        seen.append(int(kv_len[0]))
        ref, _ = A.attend_prefix(f64(q[0, T + i:T + i + 1]), f64(k[0]), f64(v[0]), T + i + 1)
        check_attention(o[0], ref, "bf16", f"step {i}")
    assert seen[:3] == [3, 4, 5] and seen[-1] == cap and int(err) == 0
    before = kc.clone()
    o = skv.attn_decode_step(q[:, cap:cap + 1].contiguous(), k[:, cap:cap + 1].contiguous(),
                             v[:, cap:cap + 1].contiguous(), kc, vc, cursor, kv_len_out=kv_len, err=err)
    torch.cuda.synchronize()
    assert int(err) == skv.DEV_CURSOR_FULL and int(cursor) == cap and int(kv_len[0]) == cap
    assert bits_equal(kc, before) and float(o.abs().sum()) == 0.0


def test_fused_step_graph_replay():
    B, Hq, Hkv, D, cap, T, steps = 1, 32, 8, 128, 1024, 60, 30
    n = T + steps
    q = SI.per_batch_normal(B, (n, Hq, D), "misc", "q", chunk=6, dtype="bf16").to(DEV)
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=6, dtype="bf16").to(DEV)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=6, dtype="bf16").to(DEV)
    kc = torch.zeros(B, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(B, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    out = torch.empty(steps, B, 1, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(skv.attn_workspace_bytes(q[:, :1], kc, kv_len=n), dtype=torch.uint8, device=DEV)
    views = [(q[:, T + i:T + i + 1], k[:, T + i:T + i + 1], v[:, T + i:T + i + 1]) for i in range(steps)]

    def job():
        cursor.zero_()
        skv.kv_cursor_advance(cursor, T, cap, idx, kv_len)
        skv.kv_write_indexed(kc, vc, k[:, :T], v[:, :T], index=idx)
        for i, (qs, ks, vs) in enumerate(views):
            skv.attn_decode_step(qs, ks, vs, kc, vc, cursor, out[i], kv_len_out=kv_len,
                                 max_seqlen_kv=n, workspace=ws)

    job()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        job()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        job()
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(out, eager), rep
        assert int(cursor) == n
        skv.attn_chunk_fwd(q[:, :1], kc, vc, kv_len=7)  # eager work between replays
        torch.cuda.synchronize()
