"""The chunk-attention tail split against the fp64 oracle: when the last round of workgroups
would leave most CU slots idle, its items are cut into key-range pieces whose partials the
last piece to arrive merges. Shapes here are chosen so that the split is planned (B=2, 8
query heads, 37 query tiles: 74 items per XCD, the last 10 cut into pieces), and the rows
checked are those of the split items (batch element 1, queries from 3456 on) plus a few
whole ones. Covered: host and device lengths, lengths so short that most pieces are empty,
causal masking, packed K/V, the full-capacity arm, fp32 output with the LSE, fp16, D=64,
a workspace reused across calls (its arrival counters return to zero), and bit-identical
results across launches and graph replays whatever the pieces' arrival order."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"

B, TQ, HQ, HKV = 2, 4700, 8, 2
SPLIT_T0 = 27 * 128  # first query of the split items (query tiles 27..36 of batch element 1)


def inputs(D, cap, dtype, seed):
    q = SI.per_batch_normal(B, (TQ, HQ, D), "misc", "q", chunk=seed, dtype=dtype)
    k = SI.per_batch_normal(B, (cap, HKV, D), "misc", "k", chunk=seed, dtype=dtype)
    v = SI.per_batch_normal(B, (cap, HKV, D), "misc", "v", chunk=seed, dtype=dtype)
    return q, k, v


def sample_rows(seed):
    rng = np.random.default_rng(seed)
    split = np.unique(np.concatenate([[SPLIT_T0, TQ - 1], rng.integers(SPLIT_T0, TQ, size=300)]))
    whole = np.unique(np.concatenate([[0], rng.integers(0, SPLIT_T0, size=20)]))
    return whole, split


def oracle_rows(q, kk, vv, ts, L, mask, Lvis=None):
    """Oracle output of query rows ts (all heads) over key rows [0, Lvis) of which [0, L) are
    active (Lvis > L only for the full-capacity arm, whose extra rows are masked)."""
    Lvis = L if Lvis is None else Lvis
    allowed = np.zeros((len(ts), Lvis), dtype=bool)
    for i, t in enumerate(ts):
        allowed[i, :L] = A.visible_keys(int(t), TQ, L, mask)
    o, lse = A.attend_keys(q[ts], kk[:Lvis], vv[:Lvis], allowed)
    return o, lse


def run(q, k, v, ws, **kw):
    return skv.attn_chunk_fwd(q, k, v, workspace=ws, **kw)


def check_split_call(dtype, D, cap, lens, mask=A.MASK_NONE, mode="host", out_f32=False, seed=0):
    q, k, v = inputs(D, cap, dtype, seed)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kw = dict(mask=mask, out_dtype=torch.float32 if out_f32 else None)
    if mode == "host":
        assert lens[0] == lens[1]
        kw["kv_len"] = lens[0]
    elif mode == "device":
        kw["kv_len_dev"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
        kw["max_seqlen_kv"] = cap
    elif mode == "full":
        kw["kv_len_dev"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
        kw["full_capacity_masked"] = True
    elif mode == "packed":
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        kd = torch.cat([kd[b, :lens[b]] for b in range(B)]).contiguous()
        vd = torch.cat([vd[b, :lens[b]] for b in range(B)]).contiguous()
        kw["cu_seqlens_kv"] = torch.from_numpy(cu).to(DEV)
        kw["max_seqlen_kv"] = max(lens)
    need = skv.attn_workspace_bytes(qd, kd, **kw)
    assert need > 0, "the tail split is not planned for this shape"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    lse = torch.empty(B, HQ, TQ, dtype=torch.float32, device=DEV)
    o = run(qd, kd, vd, ws, lse=lse, **kw)
    # the same call with a workspace too small for the split runs every item whole
    o_whole = run(qd, kd, vd, torch.zeros(16, dtype=torch.uint8, device=DEV), **kw)
    torch.cuda.synchronize()
    assert not ws[:4 * 8 * 10].any(), "arrival counters not returned to zero"

    whole, split = sample_rows(seed)
    qf, kf, vf = f64(q), f64(k), f64(v)
    got, want = [], []
    for b, ts in ((0, whole), (1, whole), (1, split)):
        L = lens[b]
        Lvis = cap if mode == "full" else None
        ref, lse_ref = oracle_rows(qf[b], kf[b], vf[b], ts, L, mask, Lvis)
        tsd = torch.from_numpy(ts).to(DEV)
        got.append(f64(o[b, tsd]))
        want.append(ref)
        if out_f32:
            assert np.max(np.abs(f64(lse[b][:, tsd]) - lse_ref)) <= 2e-3
    check_attention(np.concatenate(got), np.concatenate(want), dtype,
                    f"split {dtype} D{D} {mode} lens {lens} mask {mask}")
    # split and whole runs differ only in the order of the final sums
    diff = (o.float() - o_whole.float()).abs().max().item()
    assert diff <= (2e-3 if out_f32 else 2e-2), diff
    return ws


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_split_host_len(dtype):
    check_split_call(dtype, 128, 8192, [6500, 6500], seed=1)


def test_split_device_lens_unequal():
    check_split_call("bf16", 128, 8192, [6500, 2500], mode="device", seed=2)


def test_split_mostly_empty_pieces():
    # batch element 1 (the split items) has 100 keys: two tiles for six pieces
    check_split_call("bf16", 128, 8192, [6500, 100], mode="device", seed=3)


def test_split_causal():
    check_split_call("bf16", 128, 8192, [6500, 6500], mask=A.MASK_CAUSAL, seed=4)


def test_split_packed():
    check_split_call("bf16", 128, 6200, [6100, 5000], mode="packed", seed=5)


def test_split_full_capacity_arm():
    check_split_call("bf16", 128, 8192, [3000, 7000], mode="full", seed=6)


def test_split_fp32_out_and_lse():
    check_split_call("bf16", 128, 8192, [6500, 6500], out_f32=True, seed=7)


def test_split_d64():
    check_split_call("bf16", 64, 8192, [7000, 7000], seed=8)


def test_split_workspace_reused():
    """Back-to-back split launches on one workspace with different lengths: every launch
    merges exactly its own pieces."""
    dtype, D, cap = "bf16", 128, 8192
    q, k, v = inputs(D, cap, dtype, 9)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kl = torch.zeros(B, dtype=torch.int32, device=DEV)
    need = skv.attn_workspace_bytes(qd, kd, kv_len_dev=kl, max_seqlen_kv=cap)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    whole, split = sample_rows(9)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for lens in ([8000, 8000], [300, 5000], [8192, 64], [4000, 4100]):
        kl.copy_(torch.tensor(lens, dtype=torch.int32))
        o = skv.attn_chunk_fwd(qd, kd, vd, kv_len_dev=kl, max_seqlen_kv=cap, workspace=ws)
        ref, _ = oracle_rows(qf[1], kf[1], vf[1], split, lens[1], A.MASK_NONE)
        check_attention(o[1, torch.from_numpy(split).to(DEV)], ref, dtype, f"reuse {lens}")
    torch.cuda.synchronize()
    assert not ws[:4 * 8 * 10].any()


def test_split_is_deterministic_and_graph_replayable():
    """The merge folds every piece's partial in piece order, whichever piece arrives last, so
    repeated launches and replays of a captured graph give the same bits; the arrival counters
    return to zero on every replay."""
    dtype, D, cap = "bf16", 128, 8192
    q, k, v = inputs(D, cap, dtype, 10)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kl = torch.tensor([7000, 5000], dtype=torch.int32, device=DEV)
    need = skv.attn_workspace_bytes(qd, kd, kv_len_dev=kl, max_seqlen_kv=cap)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(qd)

    def call():
        skv.attn_chunk_fwd(qd, kd, vd, out, kv_len_dev=kl, max_seqlen_kv=cap, workspace=ws)

    call()
    torch.cuda.synchronize()
    first = out.clone()
    for _ in range(4):
        out.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(7.0)
        call()  # eager work between replays
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), rep
        assert not ws[:4 * 8 * 10].any(), rep
    whole, split = sample_rows(10)
    ref, _ = oracle_rows(f64(q)[1], f64(k)[1], f64(v)[1], split, 5000, A.MASK_NONE)
    check_attention(first[1, torch.from_numpy(split).to(DEV)], ref, dtype, "graph replay")


def test_workspace_shared_with_decode_calls():
    """One workspace of the largest size serves tail-split chunk calls and split-K decode
    calls in any order: every kind of call keeps its counters in the same 64 KiB area and
    leaves them at zero, and its partials after it. Each result equals the same call on a
    fresh zero-filled workspace, bit for bit."""
    q, k, v = inputs(128, 8192, "bf16", 11)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kl = torch.tensor([6000, 7000], dtype=torch.int32, device=DEV)
    fkw = dict(kv_len_dev=kl, max_seqlen_kv=8192)
    # decode: 16 batch elements x 8 KV heads, 32 query heads, 3000 keys
    Bd, Hqd, Hkvd, Ld = 16, 32, 8, 3000
    qdec = torch.randn(Bd, 1, Hqd, 128, device=DEV).to(torch.bfloat16)
    kdec = torch.randn(Bd, Ld, Hkvd, 128, device=DEV).to(torch.bfloat16)
    vdec = torch.randn(Bd, Ld, Hkvd, 128, device=DEV).to(torch.bfloat16)
    need_f = skv.attn_workspace_bytes(qd, kd, **fkw)
    need_d = skv.attn_workspace_bytes(qdec, kdec, kv_len=Ld)
    assert need_f > 0 and need_d > 0
    fresh = lambda n: torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref_f = skv.attn_chunk_fwd(qd, kd, vd, workspace=fresh(need_f), **fkw)
    ref_d = skv.attn_chunk_fwd(qdec, kdec, vdec, kv_len=Ld, workspace=fresh(need_d))
    ws = fresh(max(need_f, need_d))
    for rep in range(2):
        o_f = skv.attn_chunk_fwd(qd, kd, vd, workspace=ws, **fkw)
        o_d = skv.attn_chunk_fwd(qdec, kdec, vdec, kv_len=Ld, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o_f.view(torch.int16), ref_f.view(torch.int16)), rep
        assert torch.equal(o_d.view(torch.int16), ref_d.view(torch.int16)), rep
        assert not ws[:65536].any(), rep
