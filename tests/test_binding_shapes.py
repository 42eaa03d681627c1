"""The Python binding checks every tensor's shape against the sizes it passes to the C ABI
before calling it (the ABI takes raw pointers, so a mismatched tensor would be read or written
out of bounds on the device). These run on the CPU: the shape checks come before the device
checks, so CPU tensors of the wrong shape raise the shape error, and CPU tensors of the right
shape get as far as the device check -- no call reaches the library."""
import pytest
import torch

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)

bf = torch.bfloat16
SHAPE_WORDS = ("shape", "elements", "dimensions")


def z(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    assert any(w in str(e.value) for w in SHAPE_WORDS), str(e.value)


def reaches_device_check(fn, *a, **kw):
    with pytest.raises(ValueError, match="must be on a GPU"):
        fn(*a, **kw)


def test_write_shapes():
    kc, src = z(2, 16, 2, 64), z(2, 4, 2, 64)
    idx = torch.zeros(4, dtype=torch.int64)
    reaches_device_check(skv.kv_write_indexed, kc, kc.clone(), src, src.clone(), index=idx)
    shape_error(skv.kv_write_indexed, kc, z(2, 15, 2, 64), src, src.clone(), index=idx)  # v_cache
    shape_error(skv.kv_write_indexed, kc, kc.clone(), src, z(2, 5, 2, 64), index=idx)    # v_src
    shape_error(skv.kv_write_indexed, kc, kc.clone(), z(3, 4, 2, 64), z(3, 4, 2, 64), index=idx)  # B
    shape_error(skv.kv_write_indexed, kc, kc.clone(), z(2, 4, 2, 32), z(2, 4, 2, 32), index=idx)  # D
    shape_error(skv.kv_write_indexed, kc, kc.clone(), src, src.clone(), index=idx[:3])  # index
    shape_error(skv.kv_write_indexed, z(2, 16, 128), None, src, None)                   # rank
    inv = torch.zeros(32, dtype=torch.float64)
    shape_error(skv.kv_write_indexed_rope, kc, kc.clone(), src, src.clone(), inv, index=idx[:2])


def test_cursor_roll_pack_shapes():
    cur = torch.zeros(1, dtype=torch.int32)
    shape_error(skv.kv_cursor_advance, cur, 8, 64, torch.zeros(7, dtype=torch.int64))
    reaches_device_check(skv.kv_cursor_advance, cur, 8, 64, torch.zeros(8, dtype=torch.int64))
    st = z(2, 32, 2, 64)
    shape_error(skv.kv_roll_left, st, z(2, 31, 2, 64), 4, 8)
    reaches_device_check(skv.kv_roll_left, st, st.clone(), 4, 8)
    lens = torch.zeros(2, dtype=torch.int32)
    shape_error(skv.kv_ragged_metadata, lens, 16, torch.zeros(2, dtype=torch.int32))
    pad, pk = z(2, 16, 2, 64), z(20, 2, 64)
    cu = torch.zeros(3, dtype=torch.int32)
    reaches_device_check(skv.kv_pack_ragged, pad, pad.clone(), cu, pk, pk.clone())
    shape_error(skv.kv_pack_ragged, pad, pad.clone(), cu[:2], pk, pk.clone())           # cu
    shape_error(skv.kv_pack_ragged, pad, pad.clone(), cu, z(20, 2, 32), z(20, 2, 32))   # D
    shape_error(skv.kv_pack_ragged, pad, pad.clone(), cu, pk, z(19, 2, 64))             # v_packed
    shape_error(skv.kv_pack_ragged, pad, z(2, 15, 2, 64), cu, pk, pk.clone())           # v_padded


def test_ring_shapes():
    st = z(2, 3 * 16, 2, 64)
    shape_error(skv.Ring, st, z(2, 48, 2, 32), 16, 3, 1)
    reaches_device_check(skv.Ring, st, st.clone(), 16, 3, 1)


def test_attention_shapes():
    q, k = z(2, 8, 4, 128), z(2, 64, 2, 128)
    reaches_device_check(skv.attn_chunk_fwd, q, k, k.clone(), kv_len=32)
    shape_error(skv.attn_chunk_fwd, q, k, z(2, 63, 2, 128), kv_len=32)                  # v vs k
    shape_error(skv.attn_chunk_fwd, q, z(3, 64, 2, 128), z(3, 64, 2, 128), kv_len=32)   # batch
    shape_error(skv.attn_chunk_fwd, q, z(2, 64, 2, 64), z(2, 64, 2, 64), kv_len=32)     # head dim
    shape_error(skv.attn_chunk_fwd, q, k, k.clone(), z(2, 8, 4, 127), kv_len=32)        # out
    shape_error(skv.attn_chunk_fwd, q, k, k.clone(), lse=z(2, 4, 7, dtype=torch.float32), kv_len=32)
    shape_error(skv.attn_chunk_fwd, q, k, k.clone(), kv_len_dev=torch.zeros(3, dtype=torch.int32))
    pk = z(100, 2, 128)
    reaches_device_check(skv.attn_chunk_fwd, q, pk, pk.clone(), cu_seqlens_kv=torch.zeros(3, dtype=torch.int32))
    shape_error(skv.attn_chunk_fwd, q, pk, pk.clone(), cu_seqlens_kv=torch.zeros(2, dtype=torch.int32))
    shape_error(skv.attn_chunk_fwd, q, z(100, 2, 64), z(100, 2, 64), cu_seqlens_kv=torch.zeros(3, dtype=torch.int32))
    shape_error(skv.attn_chunk_fwd, q, k, k.clone(), err=torch.zeros(0, dtype=torch.int32), kv_len=32)


def test_decode_step_shapes():
    q, kc = z(1, 1, 8, 128), z(1, 256, 2, 128)
    kn, cur = z(1, 1, 2, 128), torch.zeros(1, dtype=torch.int32)
    reaches_device_check(skv.attn_decode_step, q, kn, kn.clone(), kc, kc.clone(), cur)
    shape_error(skv.attn_decode_step, q, z(1, 2, 2, 128), kn, kc, kc.clone(), cur)         # k_new
    shape_error(skv.attn_decode_step, q, kn, kn.clone(), kc, z(1, 255, 2, 128), cur)       # v_cache
    shape_error(skv.attn_decode_step, q, kn, kn.clone(), z(2, 256, 2, 128), z(2, 256, 2, 128), cur)
    shape_error(skv.attn_decode_step, q, kn, kn.clone(), kc, kc.clone(), cur,
                kv_len_out=torch.zeros(2, dtype=torch.int32))
    shape_error(skv.attn_decode_step, q, kn, kn.clone(), kc, kc.clone(), torch.zeros(0, dtype=torch.int32))
    shape_error(skv.attn_decode_step, q, kn, kn.clone(), kc, kc.clone(), cur, out=z(1, 1, 8, 64))


def test_invalid_workspace_query_raises():
    q, k = z(1, 1, 4, 128), z(1, 64, 2, 128)
    assert skv.attn_workspace_bytes(q, k, kv_len=64) > 0
    with pytest.raises(ValueError, match="kv_len"):
        skv.attn_workspace_bytes(q, k, kv_len=65)
