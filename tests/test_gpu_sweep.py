"""A seeded sweep of attention shapes against the fp64 oracle, beyond the hand-picked cases:
60 configurations drawn once from a fixed generator over batch size, query count (decode and
chunk sizes, ragged tails), GQA ratio (1-8), head dim (64, 128), the three masks (block sizes
4-64), the three addressing modes (host length, device lengths per batch element, packed
cu_seqlens_kv) and the three dtypes. Every configuration is valid by construction (a masked
row sees at least one key: lengths >= Tq), so each must meet the parity bar and return the
oracle's LSE (fp32 1e-5, bf16/fp16 2e-3)."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CONFIGS = 60


def _configs():
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(N_CONFIGS):
        dtype = ["f32", "bf16", "f16"][i % 3]
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 4))
        Tq = int(rng.choice([1, 2, 3, 4])) if rng.random() < 0.3 else int(rng.integers(5, 261))
        mask = int(rng.choice([A.MASK_NONE, A.MASK_CAUSAL, A.MASK_BLOCK_CAUSAL]))
        block = int(rng.choice([4, 16, 64])) if mask == A.MASK_BLOCK_CAUSAL else 1
        mode = ["host", "device", "packed"][int(rng.integers(0, 3))]
        lo = Tq if mask != A.MASK_NONE else 1
        lens = [int(rng.integers(lo, lo + 400)) for _ in range(B)]
        if mode == "host":
            lens = [lens[0]] * B
        cap = max(lens) + int(rng.integers(0, 70))
        out.append((i, dtype, D, Hkv, group, B, Tq, mask, block, mode, lens, cap))
    return out


@pytest.mark.parametrize("cfg", _configs(), ids=lambda c: f"c{c[0]}-{c[1]}-{c[9]}")
def test_sweep_against_oracle(cfg):
    i, dtype, D, Hkv, group, B, Tq, mask, block, mode, lens, cap = cfg
    Hq = Hkv * group
    q = SI.per_batch_normal(B, (Tq, Hq, D), "misc", "q", chunk=300 + i, dtype=dtype)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    kw = dict(mask=mask, mask_block=block, lse=lse)
    if mode == "packed":
        total = sum(lens)
        k = SI.round_to(SI.normal_f32((total, Hkv, D), SI.seed_key("misc", "k", 0, 300 + i)), dtype)
        v = SI.round_to(SI.normal_f32((total, Hkv, D), SI.seed_key("misc", "v", 0, 300 + i)), dtype)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cu_seqlens_kv=torch.from_numpy(cu).to(DEV),
                               max_seqlen_kv=max(lens), **kw)
        o_ref, lse_ref = A.attend_packed(f64(q), f64(k), f64(v), cu, mask, block)
    else:
        k = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "k", chunk=300 + i, dtype=dtype)
        v = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "v", chunk=300 + i, dtype=dtype)
        if mode == "host":
            o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len=lens[0], **kw)
        else:
            kvl = torch.tensor(lens, dtype=torch.int32, device=DEV)
            o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len_dev=kvl, max_seqlen_kv=max(lens), **kw)
        o_ref, lse_ref = A.attend_batch_prefix(f64(q), f64(k), f64(v), lens, mask, block)
    check_attention(o, o_ref, dtype, f"config {cfg}")
    tol = 1e-5 if dtype == "f32" else 2e-3
    err = float(np.max(np.abs(f64(lse) - lse_ref)))
    assert err <= tol, f"config {cfg}: lse max abs err {err:.3g}"
