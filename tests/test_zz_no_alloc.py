"""attn_decode_step_static (the fused decode step whose split-K scratch is a static array the
library holds per GPU, for callers that cannot allocate) against attn_decode_step with a
caller workspace: same outputs, caches and cursors bit for bit, and the oracle's bar, on two
configurations in a row, the second smaller than the first."""
import ctypes

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


def _run_pair(B, Hq, Hkv, D, cap, T, steps, bound, dtype, chunk):
    n = T + steps
    q = SI.per_batch_normal(B, (n, Hq, D), "misc", "q", chunk=chunk, dtype=dtype).to(DEV)
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=chunk, dtype=dtype).to(DEV)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=chunk, dtype=dtype).to(DEV)
    caches, cursors, lens, outs = [], [], [], []
    for _ in range(2):
        kc = torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV)
        vc = torch.zeros_like(kc)
        kc[:, :T], vc[:, :T] = k[:, :T], v[:, :T]
        caches.append((kc, vc))
        cursors.append(torch.full((1,), T, dtype=torch.int32, device=DEV))
        lens.append(torch.zeros(B, dtype=torch.int32, device=DEV))
        outs.append(torch.empty(steps, B, 1, Hq, D, dtype=TD[dtype], device=DEV))
    ws = torch.zeros(skv.attn_workspace_bytes(q[:, :1], caches[0][0], kv_len=bound, max_seqlen_kv=bound),
                     dtype=torch.uint8, device=DEV)
    err = torch.zeros(2, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    for i in range(steps):
        s = T + i
        args = [x[:, s:s + 1].contiguous() for x in (q, k, v)]
        skv.attn_decode_step(*args, *caches[0], cursors[0], outs[0][i], kv_len_out=lens[0],
                             max_seqlen_kv=bound, workspace=ws, err=err[:1])
        skv.attn_decode_step(*args, *caches[1], cursors[1], outs[1][i], kv_len_out=lens[1],
                             max_seqlen_kv=bound, err=err[1:], static_scratch=True)
    torch.cuda.synchronize()
    assert err.tolist() == [0, 0]
    assert bits_equal(outs[0], outs[1])
    assert bits_equal(caches[0][0], caches[1][0]) and bits_equal(caches[0][1], caches[1][1])
    assert int(cursors[1]) == n and lens[1].tolist() == [n] * B
    kf, vf, qf = f64(k), f64(v), f64(q)
    got, want = [], []
    for i in range(steps):
        for b in range(B):
            ref, _ = A.attend_prefix(qf[b, T + i:T + i + 1], kf[b], vf[b], T + i + 1)
            got.append(f64(outs[1][i, b]))
            want.append(ref)
    check_attention(np.stack(got), np.stack(want), dtype, "static-scratch decode steps")


def test_static_scratch_decode_step_equals_workspace_entry_point():
    # the decode workload's heads and key bound (20 one-chunk splits per head) ...
    _run_pair(B=1, Hq=32, Hkv=8, D=128, cap=2048, T=234, steps=12, bound=1258, dtype="bf16", chunk=91)
    # ... then a smaller call on the same scratch: fewer heads and splits, D = 64, fp16
    _run_pair(B=2, Hq=8, Hkv=2, D=64, cap=300, T=20, steps=6, bound=300, dtype="f16", chunk=92)


def test_static_scratch_refuses_a_step_larger_than_it():
    B, Hq, Hkv, D, cap = 64, 64, 8, 128, 32768  # one split per head, 64 KiB + 512 partials > 4 MiB
    q = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros(B, 1, Hkv, D, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, 64, Hkv, D, dtype=torch.bfloat16, device=DEV)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = skv.make_params(q, kc, max_seqlen_kv=0)
    p.cap = cap  # sizes only: the host check refuses before anything is read or launched
    st = skv.lib.attn_decode_step_static(q.data_ptr(), kn.data_ptr(), kn.data_ptr(), kc.data_ptr(),
                                         kc.data_ptr(), q.data_ptr(), None, cursor.data_ptr(), None,
                                         ctypes.byref(p), None)
    assert st == skv.SKV_ERR_RANGE and "static scratch" in skv.lib.skv_last_error().decode()
    assert int(cursor) == 0
