"""GPU parity of the comparison-arm roll-left and of ragged K/V packing, bit for bit against the
oracle (oracle.cache.roll_left / RollingChronological, oracle.ragged), plus the device error
bits and the packed == seqused == oracle chain at the ragged cross-attention sizes."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from oracle import cache as Cc
from oracle import ragged as R
from tests.helpers import check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t: torch.Tensor) -> np.ndarray:
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().cpu().contiguous().view(view).numpy()


@pytest.mark.parametrize("rows,sink,shift", [(10, 2, 3), (12, 0, 4), (35, 5, 5), (9, 1, 7), (64, 3, 1), (6, 0, 6)])
@pytest.mark.parametrize("dtype,Hkv,D", [(torch.float32, 2, 64), (torch.bfloat16, 3, 128)])
def test_roll_left_matches_oracle(rows, sink, shift, dtype, Hkv, D):
    """Overlapping moves (moved rows > shift), single pieces, a partial last piece, shift 1;
    K only and K+V; a canary band after the storage catches stray writes."""
    B = 2
    x = SI.per_batch_normal(B, (rows, Hkv, D), "misc", "extra", chunk=500 + rows).to(dtype)
    guard = 64
    kbuf = torch.full((B * rows * Hkv * D + guard,), 5.0, dtype=dtype, device=DEV)
    k = kbuf[:B * rows * Hkv * D].view(B, rows, Hkv, D)
    k.copy_(x.to(DEV))
    v = (x.to(DEV) * 2).contiguous()
    skv.kv_roll_left(k, v, sink, shift)
    skv.kv_roll_left(k, None, 0, rows)  # shift = rows: nothing moves
    torch.cuda.synchronize()
    for b in range(B):
        ref = Cc.roll_left(_bits(x[b]), sink, shift, rows)
        assert np.array_equal(_bits(k[b]), ref)
        ref_v = Cc.roll_left(_bits((x[b] * 2).to(dtype)), sink, shift, rows)
        assert np.array_equal(_bits(v[b]), ref_v)
    assert bool((kbuf[-guard:] == 5).all())


@pytest.mark.parametrize("n_slots,sink,C", [(7, 1, 3), (4, 0, 2), (5, 2, 1)])
def test_rolling_lifecycle_matches_oracle_and_ring_attention(n_slots, sink, C):
    """The chronological cache driven on the device (roll when full, then write the new chunk at
    the end; rewrites overwrite the newest chunk) equals RollingChronological after every write,
    and attention over it equals attention over the ring's physical order."""
    B, Hkv, Hq, D = 2, 2, 4, 64
    rows = n_slots * C
    kc = torch.zeros(B, rows, Hkv, D, dtype=torch.float32, device=DEV)
    vc = torch.zeros_like(kc)
    sims = [(Cc.RollingChronological(n_slots, sink, C, (Hkv, D)), Cc.RollingChronological(n_slots, sink, C, (Hkv, D)))
            for _ in range(B)]
    filled = 0
    for c in range(2 * n_slots + 1):
        new_chunk = True
        for r in range(1 + c % 3):
            ks = SI.per_batch_normal(B, (C, Hkv, D), "misc", "k", chunk=600 + c, rewrite=r)
            vs = SI.per_batch_normal(B, (C, Hkv, D), "misc", "v", chunk=600 + c, rewrite=r)
            if new_chunk:
                if filled + C > rows:
                    skv.kv_roll_left(kc, vc, sink * C, C)
                else:
                    filled += C
                for sk, sv in sims:
                    sk.reserve()
                    sv.reserve()
                new_chunk = False
            skv.kv_write_indexed(kc, vc, ks.to(DEV), vs.to(DEV), start=filled - C)
            for b, (sk, sv) in enumerate(sims):
                sk.write(ks[b].numpy())
                sv.write(vs[b].numpy())
            torch.cuda.synchronize()
            for b, (sk, sv) in enumerate(sims):
                assert sk.filled == filled
                np.testing.assert_array_equal(kc[b, :filled].cpu().numpy(), sk.valid())
                np.testing.assert_array_equal(vc[b, :filled].cpu().numpy(), sv.valid())
    # attention over the chronological buffer equals the oracle's (fp32, 1e-5)
    q = SI.per_batch_normal(B, (C, Hq, D), "misc", "q", chunk=700).to(DEV)
    o = skv.attn_chunk_fwd(q, kc, vc, kv_len=filled)
    ref = np.stack([A.attend_prefix(f64(q[b]), sims[b][0].valid(), sims[b][1].valid(), filled)[0] for b in range(B)])
    check_attention(o, ref, "f32", "rolling buffer attention")


@pytest.mark.parametrize("lens,max_kv", [((512, 448), 512), ((512, 51), 512), ((37, 0, 5), 37), ((1, 1), 3), ((0, 0), 4)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_metadata_and_pack_match_oracle(lens, max_kv, dtype):
    B, Hkv, D = len(lens), 3, 64
    pad_k = SI.per_batch_normal(B, (max_kv, Hkv, D), "misc", "k", chunk=800 + max_kv).to(dtype).to(DEV)
    pad_v = SI.per_batch_normal(B, (max_kv, Hkv, D), "misc", "v", chunk=800 + max_kv).to(dtype).to(DEV)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    cu = skv.kv_ragged_metadata(lens_d, max_kv)
    ref_cu, _ = R.ragged_metadata(lens)
    torch.cuda.synchronize()
    assert cu.cpu().tolist() == ref_cu.tolist()
    total = int(ref_cu[-1])
    guard = 32
    kbuf = torch.full(((total + guard) * Hkv * D,), 9.0, dtype=dtype, device=DEV)
    k_p = kbuf[:total * Hkv * D].view(total, Hkv, D)
    v_p = torch.zeros(total, Hkv, D, dtype=dtype, device=DEV)
    skv.kv_pack_ragged(pad_k, pad_v, cu, k_p, v_p)
    torch.cuda.synchronize()
    ref_k, _ = R.pack_ragged(_bits(pad_k.cpu()), lens)
    ref_v, _ = R.pack_ragged(_bits(pad_v.cpu()), lens)
    assert np.array_equal(_bits(k_p), ref_k) and np.array_equal(_bits(v_p), ref_v)
    assert bool((kbuf[total * Hkv * D:] == 9).all())


def test_pack_and_metadata_device_errors():
    B, max_kv, Hkv, D = 2, 8, 1, 64
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = torch.tensor([3, 9], dtype=torch.int32, device=DEV)  # 9 > max_kv
    cu = skv.kv_ragged_metadata(lens, max_kv, err=err)
    torch.cuda.synchronize()
    assert cu.cpu().tolist() == [0, 3, 3] and int(err.item()) & skv.DEV_KV_LEN
    err.zero_()
    pad = torch.ones(B, max_kv, Hkv, D, dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros(4, Hkv, D, dtype=torch.bfloat16, device=DEV)
    bad_cu = torch.tensor([0, 3, 6], dtype=torch.int32, device=DEV)  # second segment past row 4
    skv.kv_pack_ragged(pad, None, bad_cu, packed, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & skv.DEV_CU_SEQLENS
    assert bool((packed[:3] == 1).all()) and bool((packed[3:] == 0).all())  # bad segment skipped


@pytest.mark.parametrize("skew", [(512, 448), (512, 256), (512, 51)])
def test_pack_then_attention_at_ragged_sizes(skew):
    """Ragged cross-attention sizes (2 branches, 40 heads, D=128, bf16, max_kv 512; Q cut to
    4096 rows per branch): metadata + pack on the device, then packed attention equals the
    seqused arm bit for bit (same kernel, same key order) and the oracle on sampled rows."""
    W = SI.Ragged()
    Tq = 4096
    B, H, D, L = W.B, W.H, W.D, W.max_kv
    pad_k = SI.per_batch_device_normal(B, (L, H, D), "ragged", "k", DEV, "bf16", chunk=skew[1])
    pad_v = SI.per_batch_device_normal(B, (L, H, D), "ragged", "v", DEV, "bf16", chunk=skew[1])
    q = SI.per_batch_device_normal(B, (Tq, H, D), "ragged", "q", DEV, "bf16", chunk=skew[1])
    lens_d = torch.tensor(skew, dtype=torch.int32, device=DEV)
    cu = skv.kv_ragged_metadata(lens_d, L)
    total = sum(skew)
    k_p = torch.empty(total, H, D, dtype=torch.bfloat16, device=DEV)
    v_p = torch.empty_like(k_p)
    skv.kv_pack_ragged(pad_k, pad_v, cu, k_p, v_p)
    o_packed = skv.attn_chunk_fwd(q, k_p, v_p, cu_seqlens_kv=cu, max_seqlen_kv=L)
    o_seq = skv.attn_chunk_fwd(q, pad_k, pad_v, kv_len_dev=lens_d, max_seqlen_kv=L)
    torch.cuda.synchronize()
    assert torch.equal(o_packed, o_seq)
    rows = np.random.default_rng(7).choice(Tq, 256, replace=False)
    for b in range(B):
        kb, vb = f64(pad_k[b, :skew[b]]), f64(pad_v[b, :skew[b]])
        ref, _ = A.attend_prefix(f64(q[b, rows]), kb, vb, skew[b])
        check_attention(o_packed[b, rows], ref, "bf16", f"packed skew {skew} b={b}")
