"""Caches and packed buffers larger than 4 GiB: every byte offset a kernel forms for a batch
element, a slot or a packed segment that starts past 2^32 bytes is 64-bit. Each case puts the
data it checks beyond that boundary (batch element 1 of a B=2 slab whose elements are 4 GiB
each, rows near the end of the slab at ~8.6 GB, a ring whose second element starts at 4.3 GB,
a packed segment after a 2^21-row first segment) and compares it with the oracle, or bit for
bit, on the rows involved only; the rest of the buffers is never copied to the host."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import bits_equal, check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
Hq, Hkv, D = 32, 8, 128
ROW_BYTES = Hkv * D * 2  # one bf16 cache row, all KV heads


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _src(B, n, tensor, chunk):
    return SI.per_batch_normal(B, (n, Hkv, D), "misc", tensor, chunk=chunk, dtype="bf16").to(DEV)


def test_slab_rows_and_prefix_attention_past_4gib():
    """[LB] Summary (index_copy along the sequence dim) and [FS] Change (attention over the
    active prefix only), on a B=2 slab of 2^21 + 64 rows per element: element 1 starts at
    4 GiB + 128 KiB, its last rows end at ~8.6 GB."""
    B, cap, L = 2, (1 << 21) + 64, 700
    assert cap * ROW_BYTES > 1 << 32
    kc = torch.empty(B, cap, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    try:
        k0, v0 = _src(B, L, "k", 61), _src(B, L, "v", 61)
        skv.kv_write_indexed(kc, vc, k0, v0, start=0)
        # rows at the very end of each element, a canary row just before them
        n2 = 48
        k2, v2 = _src(B, n2, "k", 62), _src(B, n2, "v", 62)
        kc[:, cap - n2 - 1].fill_(7.0)
        vc[:, cap - n2 - 1].fill_(-7.0)
        idx = torch.arange(cap - n2, cap, dtype=torch.int64, device=DEV)
        skv.kv_write_indexed(kc, vc, k2, v2, index=idx)
        torch.cuda.synchronize()
        assert bits_equal(kc[:, :L], k0) and bits_equal(vc[:, :L], v0)
        assert bits_equal(kc[:, cap - n2:], k2) and bits_equal(vc[:, cap - n2:], v2)
        assert bool((kc[:, cap - n2 - 1] == 7.0).all()) and bool((vc[:, cap - n2 - 1] == -7.0).all())

        kp, vp = kc[:, :L].cpu(), vc[:, :L].cpu()  # every row attention may read
        lens = [L - 173, L]
        kvl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        # chunk attention (flash path): two query tiles with a ragged tail
        q = SI.per_batch_normal(B, (160, Hq, D), "misc", "q", chunk=63, dtype="bf16")
        o = skv.attn_chunk_fwd(q.to(DEV), kc, vc, kv_len_dev=kvl, max_seqlen_kv=L)
        o_ref, _ = A.attend_batch_prefix(f64(q), f64(kp), f64(vp), lens)
        check_attention(o, o_ref, "bf16", "chunk attention past 4 GiB")
        # single-token decode (split-K path)
        q1 = SI.per_batch_normal(B, (1, Hq, D), "misc", "q", chunk=64, dtype="bf16")
        o1 = skv.attn_chunk_fwd(q1.to(DEV), kc, vc, kv_len_dev=kvl, max_seqlen_kv=L)
        o1_ref, _ = A.attend_batch_prefix(f64(q1), f64(kp), f64(vp), lens)
        check_attention(o1, o1_ref, "bf16", "decode attention past 4 GiB")

        # fused decode step: writes row L of each element (element 1's at 4 GiB + 1.5 MB) and
        # attends over L + 1 keys
        cursor = torch.tensor([L], dtype=torch.int32, device=DEV)
        kn, vn = _src(B, 1, "k", 65), _src(B, 1, "v", 65)
        q2 = SI.per_batch_normal(B, (1, Hq, D), "misc", "q", chunk=65, dtype="bf16")
        o2 = skv.attn_decode_step(q2.to(DEV), kn, vn, kc, vc, cursor, max_seqlen_kv=L + 1)
        torch.cuda.synchronize()
        assert int(cursor[0]) == L + 1
        assert bits_equal(kc[:, L:L + 1], kn) and bits_equal(vc[:, L:L + 1], vn)
        kp2 = torch.cat([kp, kn.cpu()], dim=1)
        vp2 = torch.cat([vp, vn.cpu()], dim=1)
        o2_ref, _ = A.attend_batch_prefix(f64(q2), f64(kp2), f64(vp2), [L + 1, L + 1])
        check_attention(o2, o2_ref, "bf16", "fused decode step past 4 GiB")
    finally:
        del kc, vc
        _free()


def test_packed_segment_past_4gib():
    """[TR] Description: K/V packed by cu_seqlens_kv, the second segment starting past 4 GiB.
    The first segment (2^21 + 5 zero rows) gives scores of exactly 0 against zero values, so
    its output is exactly 0; the second is compared with the oracle."""
    s1, n1, Tq = (1 << 21) + 5, 700, 64
    assert s1 * ROW_BYTES > 1 << 32
    P = s1 + n1
    kp = torch.zeros(P, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    try:
        kseg = SI.round_to(SI.normal_f32((n1, Hkv, D), SI.seed_key("misc", "k", 0, 66)), "bf16")
        vseg = SI.round_to(SI.normal_f32((n1, Hkv, D), SI.seed_key("misc", "v", 0, 66)), "bf16")
        kp[s1:] = kseg.to(DEV)
        vp[s1:] = vseg.to(DEV)
        cu = torch.tensor([0, s1, P], dtype=torch.int32, device=DEV)
        q = SI.per_batch_normal(2, (Tq, Hq, D), "misc", "q", chunk=66, dtype="bf16")
        o = skv.attn_chunk_fwd(q.to(DEV), kp, vp, cu_seqlens_kv=cu, max_seqlen_kv=s1)
        torch.cuda.synchronize()
        assert bool((o[0] == 0).all())
        o_ref, _ = A.attend_packed(f64(q[1:2]), f64(kseg), f64(vseg), np.array([0, n1]))
        check_attention(o[1:2], o_ref, "bf16", "packed segment past 4 GiB")
    finally:
        del kp, vp
        _free()


def test_ring_slots_past_4gib():
    """[FD] current path / proposed boundary: a B=2 ring of 513 slots x 4096 rows per element
    (element 1 starts at 4.3 GB); two chunks written, stored bit for bit, and attention over
    the retained rows compared with the oracle."""
    B, C, n_slots, Tq, Hq_r = 2, 4096, 513, 128, 16
    rows = n_slots * C
    assert rows * ROW_BYTES > 1 << 32
    ks = torch.empty(B, rows, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vs = torch.empty_like(ks)
    ring = skv.Ring(ks, vs, C, n_slots, 1)
    try:
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        srcs = []
        for c in range(2):
            k, v = _src(B, C, "k", 70 + c), _src(B, C, "v", 70 + c)
            ring.reserve()
            ring.write(k, v, err=err)
            srcs.append((k, v))
        torch.cuda.synchronize()
        assert int(err[0]) == 0
        assert [int(x) for x in ring.kv_len] == [2 * C, 2 * C]
        for c, (k, v) in enumerate(srcs):
            assert bits_equal(ks[:, c * C:(c + 1) * C], k) and bits_equal(vs[:, c * C:(c + 1) * C], v)
        q = SI.per_batch_normal(B, (Tq, Hq_r, D), "misc", "q", chunk=72, dtype="bf16")
        o = skv.attn_chunk_fwd(q.to(DEV), ks, vs, kv_len_dev=ring.kv_len, max_seqlen_kv=rows)
        kp, vp = ks[:, :2 * C].cpu(), vs[:, :2 * C].cpu()
        o_ref, _ = A.attend_batch_prefix(f64(q[1:2]), f64(kp[1:2]), f64(vp[1:2]), [2 * C])
        check_attention(o[1:2], o_ref, "bf16", "ring element past 4 GiB")
    finally:
        ring.close()
        del ks, vs
        _free()
