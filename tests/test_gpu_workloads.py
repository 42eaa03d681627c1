"""The five synthetic workloads at their real sizes, on the GPU, against the oracle.

* tiny fp32 (H=2, D=64, capacity 64, 7 chunks of 8): everything compared, every chunk;
* decode (B=1, 32/8 heads, D=128, capacity 32768, prompt 234 + 1024 steps), fp16 and bf16:
  every output of every step and the whole written cache;
* ring (B=2, 12 heads, D=128, chunks of 4680 tokens, 7 slots with one sink, 12 chunks x 4
  rewrites, reset, 2 more chunks): storage bit-exact against the oracle's slot simulation at
  every chunk boundary and after the reset, ring metadata after every op, sampled output rows
  at every rewrite step;
* multi-user (B=8, 40 heads, capacity 16384, 16 chunks of 1024 at one shared device index,
  causal inside the chunk): sampled rows every chunk, two users' whole slabs at the end;
* ragged cross-attention (2 branches, 40 heads, Q 75600 per branch, K/V packed by
  cu_seqlens_kv at three skews): packed = seqused = padded-masked bit for bit, sampled rows.

Large inputs are drawn on the device (seeded torch generator); the oracle receives copies of
those inputs, never anything the library produced."""
import os

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from oracle import cache as Cc
from oracle import rope as R
from tests.helpers import bits_equal, check_attention, f64, report

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _bits(t):
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().cpu().contiguous().view(view).numpy()


def _from_bits(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).view(TD[dtype])


def _rope_keys_bf16_bits(k, positions, inv):
    """oracle.rope.rope_keys of k [B, T, H, D] (bf16 tensor) as bf16 bits, the heads split over
    threads (numpy releases the GIL inside its large array operations)."""
    from concurrent.futures import ThreadPoolExecutor
    kf = f64(k)
    H = kf.shape[2]
    parts = [slice(h, min(h + 2, H)) for h in range(0, H, 2)]
    with ThreadPoolExecutor(max_workers=min(len(parts), os.cpu_count() or 1, 16)) as ex:
        rot = list(ex.map(lambda sl: R.rope_keys(kf[:, :, sl], positions, inv, R.LAYOUT_HALF, "bf16"), parts))
    return _bits(torch.from_numpy(np.concatenate(rot, axis=2)).to(torch.bfloat16))


# ----------------------------------------------------------------------------------- tiny
def _tiny_run(B, W, qs, ks, vs, use_index=True):
    kc = torch.zeros(B, W.cap, W.H, W.D, dtype=torch.float32, device=DEV)
    vc = torch.zeros_like(kc)
    outs, caches = [], []
    for c in range(W.n_chunks):
        s = W.chunk * c
        if use_index:
            idx = torch.arange(s, s + W.chunk, dtype=torch.int64, device=DEV)
            skv.kv_write_indexed(kc, vc, ks[c].to(DEV), vs[c].to(DEV), index=idx)
        else:
            skv.kv_write_indexed(kc, vc, ks[c].to(DEV), vs[c].to(DEV), start=s)
        outs.append(skv.attn_chunk_fwd(qs[c].to(DEV), kc, vc, kv_len=s + W.chunk))
        caches.append((kc.clone(), vc.clone()))
    return outs, caches


def test_tiny_fp32_sequence_b1_b2():
    W = SI.Tiny()
    for B in (1, 2):
        qs = [SI.per_batch_normal(B, (W.chunk, W.H, W.D), "tiny", "q", chunk=c) for c in range(W.n_chunks)]
        ks = [SI.per_batch_normal(B, (W.chunk, W.H, W.D), "tiny", "k", chunk=c) for c in range(W.n_chunks)]
        vs = [SI.per_batch_normal(B, (W.chunk, W.H, W.D), "tiny", "v", chunk=c) for c in range(W.n_chunks)]
        outs, caches = _tiny_run(B, W, qs, ks, vs)
        outs_slice, caches_slice = _tiny_run(B, W, qs, ks, vs, use_index=False)
        rk = np.zeros((B, W.cap, W.H, W.D))
        rv = np.zeros_like(rk)
        for c in range(W.n_chunks):
            idx = np.arange(W.chunk * c, W.chunk * (c + 1))
            rk, _ = Cc.slab_write_indexed(rk, f64(ks[c]), idx)
            rv, _ = Cc.slab_write_indexed(rv, f64(vs[c]), idx)
            assert np.array_equal(f64(caches[c][0]), rk) and np.array_equal(f64(caches[c][1]), rv)
            o_ref, _ = A.attend_batch_prefix(f64(qs[c]), rk, rv, [W.chunk * (c + 1)] * B)
            check_attention(outs[c], o_ref, "f32", f"tiny B={B} chunk {c}")
            # index_copy form is bit-identical to the slice form
            assert bits_equal(outs[c], outs_slice[c])
            assert bits_equal(caches[c][0], caches_slice[c][0])
        if B == 2:
            # B=2 is bit-identical to two B=1 runs on the same per-user values
            for b in range(2):
                o1, c1 = _tiny_run(1, W, [q[b:b + 1] for q in qs], [k[b:b + 1] for k in ks],
                                   [v[b:b + 1] for v in vs])
                for c in range(W.n_chunks):
                    assert bits_equal(o1[c][0], outs[c][b])
                    assert bits_equal(c1[c][0][0], caches[c][0][b])


# --------------------------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_prefill_and_1024_steps(dtype):
    W = SI.Decode()
    n = W.prompt + W.steps
    q = SI.per_batch_normal(1, (n, W.Hq, W.D), "decode", "q", std=W.std, dtype=dtype)[0]
    k = SI.per_batch_normal(1, (n, W.Hkv, W.D), "decode", "k", std=W.std, dtype=dtype)[0]
    v = SI.per_batch_normal(1, (n, W.Hkv, W.D), "decode", "v", std=W.std, dtype=dtype)[0]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kc = torch.zeros(1, W.cap, W.Hkv, W.D, dtype=TD[dtype], device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.empty(W.prompt, dtype=torch.int64, device=DEV)
    T = W.prompt
    skv.kv_cursor_advance(cursor, T, W.cap, idx, kv_len, err)
    skv.kv_write_indexed(kc, vc, kd[None, :T], vd[None, :T], index=idx, err=err)
    o_pre = skv.attn_chunk_fwd(qd[None, :T], kc, vc, kv_len_dev=kv_len, mask=A.MASK_CAUSAL,
                               max_seqlen_kv=W.cap, err=err)
    one = torch.empty(1, dtype=torch.int64, device=DEV)
    ws = torch.zeros(skv.attn_workspace_bytes(qd[None, T:T + 1], kc, kv_len_dev=kv_len,
                                              max_seqlen_kv=W.cap), dtype=torch.uint8, device=DEV)
    outs = torch.empty(W.steps, W.Hq, W.D, dtype=TD[dtype], device=DEV)
    full_arm = {}
    for i in range(W.steps):
        skv.kv_cursor_advance(cursor, 1, W.cap, one, kv_len, err)
        skv.kv_write_indexed(kc, vc, kd[None, T + i:T + i + 1], vd[None, T + i:T + i + 1], index=one, err=err)
        skv.attn_chunk_fwd(qd[None, T + i:T + i + 1], kc, vc, outs[i][None, None], kv_len_dev=kv_len,
                           max_seqlen_kv=W.cap, workspace=ws, err=err)
        if i in (0, 511, W.steps - 1):
            full_arm[i] = skv.attn_chunk_fwd(qd[None, T + i:T + i + 1], kc, vc, kv_len_dev=kv_len,
                                             full_capacity_masked=True, err=err)
    torch.cuda.synchronize()
    assert int(err) == 0 and int(kv_len) == n and int(cursor) == n
    kf, vf = f64(k), f64(v)
    # the whole cache: rows [0, n) hold the written rows, the rest is untouched zeros
    assert np.array_equal(f64(kc[0, :n]), kf) and np.array_equal(f64(vc[0, :n]), vf)
    assert int(kc[0, n:].abs().sum()) == 0 and int(vc[0, n:].abs().sum()) == 0
    o_ref, _ = A.attend_prefix(f64(q[:T]), kf, vf, T, A.MASK_CAUSAL)
    check_attention(o_pre[0], o_ref, dtype, "prefill")
    refs = np.stack([A.attend_prefix(f64(q[T + i:T + i + 1]), kf, vf, T + i + 1)[0][0]
                     for i in range(W.steps)])
    stats = check_attention(outs, refs, dtype, "decode steps")
    for i, o in full_arm.items():
        check_attention(o[0, 0], refs[i], dtype, f"full-capacity arm step {i}")
    report(f"decode job {dtype}", stats)


# ----------------------------------------------------------------------------------- ring
def test_ring_sequence_full_size():
    W = SI.Ring()
    rows = W.n_slots * W.C
    k_store = torch.zeros(W.B, rows, W.H, W.D, dtype=torch.bfloat16, device=DEV)
    v_store = torch.zeros_like(k_store)
    ring = skv.Ring(k_store, v_store, W.C, W.n_slots, W.sink)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sims_k = [Cc.RingPhysical(W.n_slots, W.sink, W.C, (W.H, W.D), dtype=np.int16) for _ in range(W.B)]
    sims_v = [Cc.RingPhysical(W.n_slots, W.sink, W.C, (W.H, W.D), dtype=np.int16) for _ in range(W.B)]
    rng = np.random.default_rng(3)
    got, want = [], []
    # keys rotated at their absolute positions as they are written (the workload's RoPE-before-
    # write); the simulated storage holds the oracle's rotation of the same inputs
    inv = 10000.0 ** (-np.arange(W.D // 2) * 2.0 / W.D)
    inv_dev = torch.from_numpy(inv).to(DEV)
    plan = [(0, c) for c in range(W.n_chunks)] + [("reset", None)] + [(1, c) for c in range(2)]
    for seg, c in plan:
        if seg == "reset":
            ring.reset()
            for s in sims_k + sims_v:
                s.reset()
            torch.cuda.synchronize()
            assert ring.kv_len.tolist() == [0, 0] and ring.slot.tolist() == [-1, -1]
            continue
        ring.reserve()
        for s in sims_k + sims_v:
            s.reserve()
        chunk_id = 100 * seg + c
        for r in range(W.rewrites):
            shape = (W.C, W.H, W.D)
            q = SI.per_batch_device_normal(W.B, shape, "ring", "q", DEV, "bf16", chunk=chunk_id, rewrite=r)
            k = SI.per_batch_device_normal(W.B, shape, "ring", "k", DEV, "bf16", chunk=chunk_id, rewrite=r)
            v = SI.per_batch_device_normal(W.B, shape, "ring", "v", DEV, "bf16", chunk=chunk_id, rewrite=r)
            ring.write_rope(k, v, inv_dev, rope_layout=skv.ROPE_HALF, err=err)
            o = skv.attn_chunk_fwd(q, k_store, v_store, kv_len_dev=ring.kv_len, max_seqlen_kv=rows)
            heads = [int(rng.integers(W.H)) for _ in range(W.B)]
            pos = R.ring_positions(c, W.C)
            vb = _bits(v)
            if r == W.rewrites - 1:  # the retained rewrite: every head, for the storage compare
                kb = _rope_keys_bf16_bits(k, pos, inv)
            else:  # only the head the attention check samples (the others are rewritten later)
                kb = _bits(k).copy()
                for b, h in enumerate(heads):
                    kb[b, :, h:h + 1] = _rope_keys_bf16_bits(k[b:b + 1, :, h:h + 1], pos, inv)[0]
            for b in range(W.B):
                sims_k[b].write(kb[b])
                sims_v[b].write(vb[b])
            torch.cuda.synchronize()
            lens = ring.kv_len.tolist()
            assert lens == [s.valid_tokens() for s in sims_k]
            assert ring.slot.tolist() == [s.current_slot() for s in sims_k]
            # sampled rows (two (b, h) pairs x 192 queries, first and last query included)
            # against the oracle over the simulated storage, which was built from the inputs
            for b in range(W.B):
                h = heads[b]
                ts = np.unique(np.concatenate([[0, W.C - 1], rng.integers(W.C, size=190)]))
                L = lens[b]
                kk = f64(_from_bits(sims_k[b].storage[:L, h:h + 1], "bf16"))
                vv = f64(_from_bits(sims_v[b].storage[:L, h:h + 1], "bf16"))
                tsd = torch.from_numpy(ts).to(DEV)
                ref, _ = A.attend_prefix(f64(q[b, tsd, h:h + 1]), kk, vv, L)
                og = f64(o[b, tsd, h:h + 1])
                check_attention(og, ref, "bf16", f"ring {seg}/{c}/{r} b{b} h{h}")
                got.append(og)
                want.append(ref)
        # storage bit-exact at the end of every chunk
        gk, gv = _bits(k_store), _bits(v_store)
        for b in range(W.B):
            assert np.array_equal(gk[b], sims_k[b].storage), (seg, c, b)
            assert np.array_equal(gv[b], sims_v[b].storage), (seg, c, b)
    assert int(err) == 0
    stats = check_attention(np.concatenate(got), np.concatenate(want), "bf16", "ring, all sampled rows")
    report("ring sequence", stats)


# ---------------------------------------------------------------------------- multi-user
def test_multiuser_block_causal_full_size():
    W = SI.MultiUser()
    kc = torch.zeros(W.B, W.cap, W.H, W.D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(W.B, dtype=torch.int32, device=DEV)
    idx = torch.empty(W.chunk, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(4)
    sources_k, sources_v = [], []
    got, want = [], []
    for c in range(W.n_chunks):
        shape = (W.chunk, W.H, W.D)
        q = SI.per_batch_device_normal(W.B, shape, "multiuser", "q", DEV, "bf16", chunk=c)
        k = SI.per_batch_device_normal(W.B, shape, "multiuser", "k", DEV, "bf16", chunk=c)
        v = SI.per_batch_device_normal(W.B, shape, "multiuser", "v", DEV, "bf16", chunk=c)
        skv.kv_cursor_advance(cursor, W.chunk, W.cap, idx, kv_len, err)
        skv.kv_write_indexed(kc, vc, k, v, index=idx, err=err)
        o = skv.attn_chunk_fwd(q, kc, vc, kv_len_dev=kv_len, mask=A.MASK_BLOCK_CAUSAL,
                               mask_block=W.block, max_seqlen_kv=W.cap, err=err)
        sources_k.append(k.cpu())
        sources_v.append(v.cpu())
        L = W.chunk * (c + 1)
        # one (b, h) pair per chunk, all 1024 query rows of the chunk
        b, h = int(rng.integers(W.B)), int(rng.integers(W.H))
        kk = f64(torch.cat([s[b, :, h:h + 1] for s in sources_k]))
        vv = f64(torch.cat([s[b, :, h:h + 1] for s in sources_v]))
        ref, _ = A.attend_prefix(f64(q[b, :, h:h + 1]), kk, vv, L, A.MASK_BLOCK_CAUSAL, W.block)
        og = f64(o[b, :, h:h + 1])
        check_attention(og, ref, "bf16", f"chunk {c} b{b} h{h}")
        got.append(og)
        want.append(ref)
    torch.cuda.synchronize()
    assert int(err) == 0 and kv_len.tolist() == [W.cap] * W.B
    stats = check_attention(np.concatenate(got), np.concatenate(want), "bf16", "multi-user, all sampled rows")
    report("multi-user sequence", stats)
    for b in (0, W.B - 1):
        ref_k = np.zeros((1, W.cap, W.H, W.D), dtype=np.int16)
        for c in range(W.n_chunks):
            ref_k, _ = Cc.slab_write_indexed(ref_k, _bits(sources_k[c][b:b + 1]),
                                             np.arange(W.chunk * c, W.chunk * (c + 1)))
        assert np.array_equal(_bits(kc[b:b + 1]), ref_k)


# -------------------------------------------------------------------------------- ragged
@pytest.mark.parametrize("lens", SI.Ragged().skews)
def test_ragged_cross_attention_full_size(lens):
    W = SI.Ragged()
    q = SI.per_batch_device_normal(W.B, (W.Tq, W.H, W.D), "ragged", "q", DEV, "bf16")
    total = sum(lens)
    kp = SI.round_to(SI.normal_f32((total, W.H, W.D), SI.seed_key("ragged", "k", 0, lens[1])), "bf16")
    vp = SI.round_to(SI.normal_f32((total, W.H, W.D), SI.seed_key("ragged", "v", 0, lens[1])), "bf16")
    cu = torch.tensor([0, lens[0], total], dtype=torch.int32)
    kpad = torch.zeros(W.B, W.max_kv, W.H, W.D, dtype=torch.bfloat16)
    vpad = torch.zeros_like(kpad)
    for b in range(W.B):
        kpad[b, :lens[b]] = kp[cu[b]:cu[b + 1]]
        vpad[b, :lens[b]] = vp[cu[b]:cu[b + 1]]
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_p = skv.attn_chunk_fwd(q, kp.to(DEV), vp.to(DEV), cu_seqlens_kv=cu.to(DEV), max_seqlen_kv=W.max_kv)
    o_s = skv.attn_chunk_fwd(q, kpad.to(DEV), vpad.to(DEV), kv_len_dev=used, max_seqlen_kv=W.max_kv)
    o_m = skv.attn_chunk_fwd(q, kpad.to(DEV), vpad.to(DEV), kv_len_dev=used, max_seqlen_kv=W.max_kv,
                             full_capacity_masked=True)
    assert bits_equal(o_p, o_s) and bits_equal(o_p, o_m)
    rng = np.random.default_rng(lens[1])
    got, want = [], []
    for _ in range(8):  # 8 (b, h) pairs x 512 query rows (first and last query included)
        b, h = int(rng.integers(W.B)), int(rng.integers(W.H))
        ts = np.unique(np.concatenate([[0, W.Tq - 1], rng.integers(W.Tq, size=510)]))
        tsd = torch.from_numpy(ts).to(DEV)
        kk = f64(kp[cu[b]:cu[b + 1], h:h + 1])
        vv = f64(vp[cu[b]:cu[b + 1], h:h + 1])
        ref, _ = A.attend_prefix(f64(q[b, tsd, h:h + 1]), kk, vv, lens[b])
        got.append(f64(o_p[b, tsd, h:h + 1]))
        want.append(ref)
    stats = check_attention(np.concatenate(got), np.concatenate(want), "bf16", f"ragged {lens}")
    report(f"ragged {lens}", stats)
