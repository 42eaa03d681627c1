"""Split-K decode merge coverage against the fp64 oracle: query rows per KV head from 1 to 16
(one to four row quads, padded quads included), head dims 64 and 128, split counts from 3 to
32 (empty splits, and the merge paths where a thread folds several batches of partials or
several (row quad, column) pairs), outputs in the input dtype and in fp32, and the LSE."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import bits_equal, check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # B, Tq, Hq, Hkv, D, kv_len, mask
    (1, 4, 8, 2, 128, 4500, A.MASK_NONE),    # 16 rows: four quads, 32 splits, two o batches
    (1, 4, 8, 2, 128, 4500, A.MASK_CAUSAL),
    (1, 2, 8, 2, 128, 4097, A.MASK_NONE),    # 8 rows, 32 splits of 192 keys: the last ten empty
    (1, 1, 6, 2, 128, 3000, A.MASK_NONE),    # 3 rows: a partly padded quad
    (2, 1, 2, 2, 64, 2000, A.MASK_NONE),     # 1 row, D = 64: four threads per (quad, column)
    (1, 3, 4, 1, 64, 2500, A.MASK_CAUSAL),   # 12 rows, D = 64
    (1, 1, 32, 8, 128, 257, A.MASK_NONE),    # the decode workload's heads, 3 splits
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_decode_merge_matches_oracle(dtype, out_f32, case):
    B, Tq, Hq, Hkv, D, kv_len, mask = case
    cap = kv_len + 3
    q = SI.per_batch_normal(B, (Tq, Hq, D), "misc", "q", chunk=41, dtype=dtype)
    k = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "k", chunk=41, dtype=dtype)
    v = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "v", chunk=41, dtype=dtype)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), lse=lse, kv_len=kv_len, mask=mask,
                           out_dtype=torch.float32 if out_f32 else None)
    o_ref, lse_ref = A.attend_batch_prefix(f64(q), f64(k), f64(v), [kv_len] * B, mask, 1)
    r = check_attention(o, o_ref, dtype, f"{case} {dtype}")
    if out_f32:
        assert o.dtype == torch.float32 and r["max_abs"] < 5e-3
    assert np.max(np.abs(f64(lse) - lse_ref)) <= 2e-3


def test_decode_merge_reuses_its_workspace():
    """Back-to-back launches on one workspace with different split counts: the arrival
    counters return to zero after each launch, so every launch merges exactly its own splits."""
    B, Tq, Hq, Hkv, D, cap = 1, 1, 8, 2, 128, 5000
    q = SI.per_batch_normal(B, (Tq, Hq, D), "misc", "q", chunk=43, dtype="bf16").to(DEV)
    k = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "k", chunk=43, dtype="bf16").to(DEV)
    v = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "v", chunk=43, dtype="bf16").to(DEV)
    ws = torch.zeros(skv.attn_workspace_bytes(q, k, kv_len=cap), dtype=torch.uint8, device=DEV)
    for kv_len in (4999, 300, 2049, 130, 4999):
        o = skv.attn_chunk_fwd(q, k, v, kv_len=kv_len, workspace=ws)
        o_ref, _ = A.attend_batch_prefix(f64(q), f64(k), f64(v), [kv_len] * B, A.MASK_NONE, 1)
        check_attention(o, o_ref, "bf16", f"kv_len {kv_len}")


@pytest.mark.parametrize("fused", [False, True])
def test_decode_lengths_below_and_past_the_bound(fused):
    """The split grid is sized from max_seqlen_kv (256 keys: four one-chunk splits, whose
    tiles are loaded before the length is read). Shorter lengths leave splits empty; they
    leave at once and the merge reads only the others. A device length past the bound makes
    every split longer than one chunk: the early tiles are dropped and the splits loaded
    again. Every step is checked against the oracle."""
    B, Hq, Hkv, D, cap, bound = 1, 32, 8, 128, 2048, 256
    q = SI.per_batch_normal(B, (1, Hq, D), "misc", "q", chunk=47, dtype="bf16").to(DEV)
    k = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "k", chunk=47, dtype="bf16").to(DEV)
    v = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "v", chunk=47, dtype="bf16").to(DEV)
    ws = torch.zeros(skv.attn_workspace_bytes(q, k, kv_len=bound), dtype=torch.uint8, device=DEV)
    kv_len = torch.zeros(B, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for L in (1, 63, 64, 65, 130, 255, 256, 257, 700, 2048):
        if fused:
            kc, vc = k.clone(), v.clone()
            cursor = torch.full((1,), L - 1, dtype=torch.int32, device=DEV)
            o = skv.attn_decode_step(q, k[:, L - 1:L].contiguous(), v[:, L - 1:L].contiguous(), kc, vc,
                                     cursor, kv_len_out=kv_len, max_seqlen_kv=bound, workspace=ws, err=err)
            torch.cuda.synchronize()
            assert int(cursor) == L and kv_len.tolist() == [L]
            assert bits_equal(kc, k) and bits_equal(vc, v)
        else:
            kv_len.fill_(L)
            o = skv.attn_chunk_fwd(q, k, v, kv_len_dev=kv_len, max_seqlen_kv=bound, workspace=ws, err=err)
        o_ref, _ = A.attend_batch_prefix(qf, kf, vf, [L], A.MASK_NONE, 1)
        check_attention(o, o_ref, "bf16", f"kv_len {L} fused {fused}")
    torch.cuda.synchronize()
    assert int(err) == 0
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0  # arrival counters back at zero
