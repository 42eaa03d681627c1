"""A seeded sweep of fused decode steps (attn_decode_step) beyond the hand-picked shapes: 24
configurations drawn once from a fixed generator over batch size, KV heads, GQA ratio and
step width (Tq * Hq/Hkv <= 16 query rows per KV head), head dim, dtype, causal or no mask,
cache capacity, prompt length (so the cursor starts anywhere in the cache) and the host key
bound (none, or the capacity). Each runs three steps; every step must equal the three-call
sequence bit for bit (output and caches) and meet the parity bar against the oracle."""
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
STEPS = 3


def _configs():
    rng = np.random.default_rng(1312)
    out = []
    for i in range(24):
        dtype = ["bf16", "f16"][i % 2]
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Tq = int(rng.integers(1, 5))
        group = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * Tq <= 16]))
        B = int(rng.integers(1, 4))
        mask = int(rng.choice([A.MASK_NONE, A.MASK_CAUSAL]))
        cap = int(rng.integers(64, 2049))
        T = int(rng.integers(Tq, cap - STEPS * Tq + 1))
        bound = int(rng.choice([0, cap]))
        out.append((i, dtype, D, Hkv, group, Tq, B, mask, cap, T, bound))
    return out


@pytest.mark.parametrize("cfg", _configs(), ids=lambda c: f"d{c[0]}-{c[1]}")
def test_decode_sweep(cfg):
    i, dtype, D, Hkv, group, Tq, B, mask, cap, T, bound = cfg
    Hq = Hkv * group
    n = T + STEPS * Tq
    q = SI.per_batch_normal(B, (n, Hq, D), "misc", "q", chunk=500 + i, dtype=dtype).to(DEV)
    k = SI.per_batch_normal(B, (n, Hkv, D), "misc", "k", chunk=500 + i, dtype=dtype).to(DEV)
    v = SI.per_batch_normal(B, (n, Hkv, D), "misc", "v", chunk=500 + i, dtype=dtype).to(DEV)
    caches = [(torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV),
               torch.zeros(B, cap, Hkv, D, dtype=TD[dtype], device=DEV)) for _ in range(2)]
    cursors = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2)]
    lens = [torch.zeros(B, dtype=torch.int32, device=DEV) for _ in range(2)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    for (kc, vc), cur, kl in zip(caches, cursors, lens):  # prefill of T rows
        skv.kv_cursor_advance(cur, T, cap, idx, kl)
        skv.kv_write_indexed(kc, vc, k[:, :T].contiguous(), v[:, :T].contiguous(), index=idx)
    one = torch.empty(Tq, dtype=torch.int64, device=DEV)
    kf, vf, qf = f64(k), f64(v), f64(q)
    got, want = [], []
    for s_i in range(STEPS):
        s = T + s_i * Tq
        qs, ks, vs = (x[:, s:s + Tq].contiguous() for x in (q, k, v))
        fused = skv.attn_decode_step(qs, ks, vs, caches[0][0], caches[0][1], cursors[0], kv_len_out=lens[0],
                                     mask=mask, max_seqlen_kv=bound, err=err)
        skv.kv_cursor_advance(cursors[1], Tq, cap, one, lens[1])
        skv.kv_write_indexed(caches[1][0], caches[1][1], ks, vs, index=one)
        three = skv.attn_chunk_fwd(qs, caches[1][0], caches[1][1], kv_len_dev=lens[1], mask=mask,
                                   max_seqlen_kv=bound)
        assert bits_equal(fused, three), (cfg, s_i)
        for b in range(B):
            ref, _ = A.attend_prefix(qf[b, s:s + Tq], kf[b], vf[b], s + Tq, mask)
            got.append(f64(fused[b]))
            want.append(ref)
    torch.cuda.synchronize()
    assert int(err) == 0, cfg
    assert bits_equal(caches[0][0], caches[1][0]) and bits_equal(caches[0][1], caches[1][1]), cfg
    assert int(cursors[0]) == n and lens[0].tolist() == [n] * B, cfg
    check_attention(np.stack(got), np.stack(want), dtype, f"config {cfg}")
