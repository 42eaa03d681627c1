"""GPU parity of attn_chunk_fwd against the fp64 oracle, element by element, at sizes the
oracle finishes in seconds that still span several query/key tiles and ragged tails:
every path (exact fp32, bf16/fp16 flash, bf16/fp16 split-K decode), every addressing mode
(host kv_len, device kv_len, packed cu_seqlens_kv, the full-capacity masked arm), every
mask, GQA, the LSE output, and the properties the pages fix (active prefix = masked full
capacity, packed = padded-masked, B=2 = two B=1 runs, determinism, poisoned tails)."""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import bits_equal, check_attention, f64

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def make(B, Tq, Hq, Hkv, D, cap, dtype, seed=0, std=1.0):
    q = SI.per_batch_normal(B, (Tq, Hq, D), "misc", "q", chunk=seed, std=std, dtype=dtype)
    k = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "k", chunk=seed, std=std, dtype=dtype)
    v = SI.per_batch_normal(B, (cap, Hkv, D), "misc", "v", chunk=seed, std=std, dtype=dtype)
    return q, k, v


def oracle_prefix(q, k, v, kv_lens, mask=A.MASK_NONE, block=1):
    o, lse = A.attend_batch_prefix(f64(q), f64(k), f64(v), kv_lens, mask, block)
    return o, lse


CASES = [
    # B, Tq, Hq, Hkv, D, cap, kv_len, mask, block
    (1, 8, 2, 2, 64, 64, 56, A.MASK_NONE, 1),
    (2, 130, 4, 2, 128, 400, 333, A.MASK_NONE, 1),
    (2, 200, 4, 1, 128, 300, 300, A.MASK_CAUSAL, 1),
    (1, 257, 2, 2, 128, 600, 513, A.MASK_CAUSAL, 1),
    (2, 192, 4, 4, 128, 700, 640, A.MASK_BLOCK_CAUSAL, 64),
    (1, 100, 3, 1, 128, 256, 190, A.MASK_BLOCK_CAUSAL, 7),
    (2, 75, 8, 2, 64, 200, 150, A.MASK_CAUSAL, 1),
    (1, 1, 32, 8, 128, 2048, 1258, A.MASK_NONE, 1),     # decode step, GQA 4:1
    (2, 3, 8, 2, 128, 512, 301, A.MASK_CAUSAL, 1),      # short causal chunk -> split-K
    (1, 4, 4, 1, 64, 300, 4, A.MASK_CAUSAL, 1),         # chunk equal to the prefix
    (1, 1, 4, 4, 128, 100, 1, A.MASK_NONE, 1),          # kv_len = 1
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("case", CASES)
def test_prefix_attention_matches_oracle(dtype, case):
    B, Tq, Hq, Hkv, D, cap, kv_len, mask, block = case
    q, k, v = make(B, Tq, Hq, Hkv, D, cap, dtype, seed=cap + Tq)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), lse=lse, kv_len=kv_len, mask=mask,
                           mask_block=block)
    o_ref, lse_ref = oracle_prefix(q, k, v, [kv_len] * B, mask, block)
    check_attention(o, o_ref, dtype, f"{case} {dtype}")
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert np.max(np.abs(f64(lse) - lse_ref)) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", [None, torch.float32])
def test_fp32_output(dtype, out_dtype):
    q, k, v = make(2, 150, 4, 2, 128, 300, dtype, seed=5)
    o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len=280, out_dtype=out_dtype)
    o_ref, _ = oracle_prefix(q, k, v, [280, 280])
    r = check_attention(o, o_ref, dtype)
    if out_dtype is torch.float32:
        assert o.dtype == torch.float32 and r["max_abs"] < 5e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Tq", [1, 96])
def test_device_kv_len_per_batch(dtype, Tq):
    B, Hq, Hkv, D, cap = 3, 4, 2, 128, 500
    q, k, v = make(B, Tq, Hq, Hkv, D, cap, dtype, seed=11)
    lens = [500, 97, 260]
    kv_len_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len_dev=kv_len_dev,
                           mask=A.MASK_CAUSAL, max_seqlen_kv=cap)
    o_ref, _ = oracle_prefix(q, k, v, lens, A.MASK_CAUSAL)
    check_attention(o, o_ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("Tq", [1, 2, 300])
def test_active_prefix_equals_full_capacity_masked_arm(dtype, Tq):
    """fish-speech #1312: active prefix = full capacity with a masked tail. On the GPU the two
    are bit-identical because fully masked tiles leave the running state untouched."""
    B, Hq, Hkv, D, cap, kv_len = 2, 8, 2, 128, 1024, 333
    q, k, v = make(B, Tq, Hq, Hkv, D, cap, dtype, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kd[:, kv_len:] = 0  # the unpopulated tail of a zero-initialised cache
    vd[:, kv_len:] = 0
    a = skv.attn_chunk_fwd(qd, kd, vd, kv_len=kv_len)
    f = skv.attn_chunk_fwd(qd, kd, vd, kv_len=kv_len, full_capacity_masked=True)
    o_ref, _ = oracle_prefix(q, k, v, [kv_len] * B)
    check_attention(a, o_ref, dtype)
    check_attention(f, o_ref, dtype)
    if Tq > 4 or dtype == "f32":
        assert bits_equal(a, f)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("Tq,lens", [(300, (512, 51)), (1, (200, 448)), (129, (64, 1))])
def test_packed_equals_padded_masked_and_oracle(dtype, Tq, lens):
    """TensorRT-LLM #18973: packed K/V (cu_seqlens_kv, padded Q) = padded K/V with a per-batch
    used length (seqused) = padded and masked = per-sample reference."""
    B, Hq, Hkv, D = 2, 4, 4, 128
    L = max(lens)
    q = SI.per_batch_normal(B, (Tq, Hq, D), "misc", "q", chunk=21, dtype=dtype)
    kp = SI.round_to(SI.normal_f32((sum(lens), Hkv, D), SI.seed_key("misc", "k", 0, 21)), dtype)
    vp = SI.round_to(SI.normal_f32((sum(lens), Hkv, D), SI.seed_key("misc", "v", 0, 21)), dtype)
    cu = torch.tensor([0, lens[0], lens[0] + lens[1]], dtype=torch.int32)
    kpad = torch.zeros(B, L, Hkv, D, dtype=TD[dtype])
    vpad = torch.zeros_like(kpad)
    for b in range(B):
        kpad[b, :lens[b]] = kp[cu[b]:cu[b + 1]]
        vpad[b, :lens[b]] = vp[cu[b]:cu[b + 1]]
    qd = q.to(DEV)
    o_packed = skv.attn_chunk_fwd(qd, kp.to(DEV), vp.to(DEV), cu_seqlens_kv=cu.to(DEV), max_seqlen_kv=L)
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_used = skv.attn_chunk_fwd(qd, kpad.to(DEV), vpad.to(DEV), kv_len_dev=used, max_seqlen_kv=L)
    o_mask = skv.attn_chunk_fwd(qd, kpad.to(DEV), vpad.to(DEV), kv_len_dev=used, max_seqlen_kv=L,
                                full_capacity_masked=True)
    o_ref, _ = A.attend_packed(f64(q), f64(kp), f64(vp), cu.numpy())
    for o in (o_packed, o_used, o_mask):
        check_attention(o, o_ref, dtype)
    assert bits_equal(o_packed, o_used)
    if Tq > 4 or dtype == "f32":
        assert bits_equal(o_packed, o_mask)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batch_of_two_equals_two_single_runs_and_determinism(dtype):
    q, k, v = make(2, 200, 4, 2, 128, 384, dtype, seed=8)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    both = skv.attn_chunk_fwd(qd, kd, vd, kv_len=384, mask=A.MASK_CAUSAL)
    again = skv.attn_chunk_fwd(qd, kd, vd, kv_len=384, mask=A.MASK_CAUSAL)
    assert bits_equal(both, again)
    for b in range(2):
        one = skv.attn_chunk_fwd(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(),
                                 vd[b:b + 1].contiguous(), kv_len=384, mask=A.MASK_CAUSAL)
        assert bits_equal(one[0], both[b])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Tq", [1, 130])
def test_poisoned_tail_is_never_read(dtype, Tq):
    """Rows past kv_len hold NaN; prefix-mode attention must not touch them."""
    q, k, v = make(1, Tq, 4, 2, 128, 512, dtype, seed=9)
    kd, vd = k.to(DEV), v.to(DEV)
    kd[:, 200:] = float("nan")
    vd[:, 200:] = float("nan")
    o = skv.attn_chunk_fwd(q.to(DEV), kd, vd, kv_len=200)
    o_ref, _ = oracle_prefix(q, k, v, [200])
    check_attention(o, o_ref, dtype)


def test_device_errors_skip_batch_elements():
    q, k, v = make(3, 64, 2, 2, 128, 128, "bf16", seed=1)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = torch.tensor([128, 0, 129], dtype=torch.int32, device=DEV)
    o = skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len_dev=lens, err=err)
    torch.cuda.synchronize()
    assert int(err) == skv.DEV_KV_LEN
    o_ref, _ = oracle_prefix(q[:1], k[:1], v[:1], [128])
    check_attention(o[:1], o_ref, "bf16")
    err.zero_()
    bad_cu = torch.tensor([0, 64, 64, 100], dtype=torch.int32, device=DEV)  # empty segment
    kp, vp = k[0, :100].contiguous().to(DEV), v[0, :100].contiguous().to(DEV)
    skv.attn_chunk_fwd(q.to(DEV), kp, vp, cu_seqlens_kv=bad_cu, err=err)
    torch.cuda.synchronize()
    assert int(err) == skv.DEV_CU_SEQLENS
    err.zero_()
    short = torch.tensor([10, 128, 128], dtype=torch.int32, device=DEV)  # causal Tq=64 > 10
    skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kv_len_dev=short, mask=A.MASK_CAUSAL, err=err)
    torch.cuda.synchronize()
    assert int(err) == skv.DEV_KV_LEN


def test_host_validation_errors():
    q, k, v = make(1, 8, 4, 2, 128, 64, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for kv_len in (0, 65):
        with pytest.raises(skv.SkvError) as e:
            skv.attn_chunk_fwd(qd, kd, vd, kv_len=kv_len)
        assert e.value.status == skv.SKV_ERR_RANGE
    skv.attn_chunk_fwd(qd, kd, vd, kv_len=1)
    skv.attn_chunk_fwd(qd, kd, vd, kv_len=64)
    with pytest.raises(skv.SkvError) as e:
        skv.attn_chunk_fwd(qd, kd, vd, kv_len=4, mask=A.MASK_CAUSAL)
    assert e.value.status == skv.SKV_ERR_RANGE
    with pytest.raises(skv.SkvError) as e:
        skv.attn_chunk_fwd(qd, kd, vd, kv_len_dev=torch.ones(1, dtype=torch.int32, device=DEV),
                           cu_seqlens_kv=torch.zeros(2, dtype=torch.int32, device=DEV))
    assert e.value.status == skv.SKV_ERR_UNSUPPORTED
    q96 = torch.zeros(1, 8, 4, 96, dtype=torch.bfloat16, device=DEV)
    k96 = torch.zeros(1, 64, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(skv.SkvError) as e:
        skv.attn_chunk_fwd(q96, k96, k96, kv_len=8)
    assert e.value.status == skv.SKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_steps_through_the_device_cursor(dtype):
    """A short prefill + decode sequence driven entirely by device metadata: the cursor
    yields the write index and kv_len; write and attention read them on the device."""
    Hq, Hkv, D, cap, T, steps = 8, 2, 128, 256, 37, 20
    rng_q = SI.per_batch_normal(1, (T + steps, Hq, D), "misc", "q", chunk=77, dtype=dtype)
    rng_k = SI.per_batch_normal(1, (T + steps, Hkv, D), "misc", "k", chunk=77, dtype=dtype)
    rng_v = SI.per_batch_normal(1, (T + steps, Hkv, D), "misc", "v", chunk=77, dtype=dtype)
    kc = torch.zeros(1, cap, Hkv, D, dtype=TD[dtype], device=DEV)
    vc = torch.zeros_like(kc)
    cursor = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.empty(T, dtype=torch.int64, device=DEV)
    skv.kv_cursor_advance(cursor, T, cap, idx, kv_len)
    skv.kv_write_indexed(kc, vc, rng_k[:, :T].contiguous().to(DEV), rng_v[:, :T].contiguous().to(DEV), index=idx)
    o = skv.attn_chunk_fwd(rng_q[:, :T].contiguous().to(DEV), kc, vc, kv_len_dev=kv_len,
                           mask=A.MASK_CAUSAL, max_seqlen_kv=cap)
    kref, vref = f64(rng_k), f64(rng_v)
    o_ref, _ = A.attend_prefix(f64(rng_q[0, :T]), kref[0], vref[0], T, A.MASK_CAUSAL)
    check_attention(o[0], o_ref, dtype)
    one = torch.empty(1, dtype=torch.int64, device=DEV)
    for i in range(steps):
        skv.kv_cursor_advance(cursor, 1, cap, one, kv_len)
        skv.kv_write_indexed(kc, vc, rng_k[:, T + i:T + i + 1].contiguous().to(DEV),
                             rng_v[:, T + i:T + i + 1].contiguous().to(DEV), index=one)
        o = skv.attn_chunk_fwd(rng_q[:, T + i:T + i + 1].contiguous().to(DEV), kc, vc,
                               kv_len_dev=kv_len, max_seqlen_kv=cap)
        o_ref, _ = A.attend_prefix(f64(rng_q[0, T + i:T + i + 1]), kref[0], vref[0], T + i + 1)
        check_attention(o[0], o_ref, dtype, f"step {i}")
    assert int(kv_len) == T + steps


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", [None, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
def test_output_rows_stay_inside_out(dtype, out_dtype, D):
    """Outputs leave as whole rows, 32 per wavefront: with Tq = 37 the second wavefront of a
    query tile has 5 rows and the last two none. Every output row matches the oracle and the
    NaN canaries on both sides of `out` (one extra query row of every head) stay untouched."""
    B, Tq, Hq, Hkv, cap, kv_len = 2, 37, 3, 1, 200, 170
    q, k, v = make(B, Tq, Hq, Hkv, D, cap, dtype, seed=D + 11)
    ot = out_dtype or TD[dtype]
    pad = Hq * D  # one query row of all heads
    n = B * Tq * Hq * D
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=ot, device=DEV)
    out = buf[pad:pad + n].view(B, Tq, Hq, D)
    skv.attn_chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, kv_len=kv_len, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, _ = oracle_prefix(q, k, v, [kv_len] * B)
    check_attention(out, o_ref, dtype, f"D={D} out={ot}")
    assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + n:]).all(), "write outside out"
