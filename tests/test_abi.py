"""C-ABI checks that need no GPU: the library loads and exports every function include/skv.h
declares, the ctypes mirror of skv_attn_params has the C layout (offsets from gcc), and every
host-checkable error returns its status before anything is launched (fake device pointers
are never dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skv.h")

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
lib = skv.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_every_declared_function_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by libskv.so"
    assert set(names) == set(skv.EXPORTED)


def test_params_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in skv.skv_attn_params._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"skv.h\"\nint main(void){\n"
                   + "".join(f'printf("%zu\\n", offsetof(skv_attn_params, {f}));\n' for f in fields)
                   + 'printf("%zu\\n", sizeof(skv_attn_params));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    py = [getattr(skv.skv_attn_params, f).offset for f in fields] + [ctypes.sizeof(skv.skv_attn_params)]
    assert out == py


# fake, 16-byte aligned "device" addresses: validation fails before any of them is used
P = 0x10000
BAD = 0x10008  # 8-byte aligned only


def params(**kw):
    p = skv.skv_attn_params()
    base = dict(B=1, Tq=8, Hq=4, Hkv=2, D=128, dtype=skv.SKV_BF16, out_dtype=skv.SKV_BF16, cap=64,
                kv_len=32, mask=0, mask_block=1, scale=0.0)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def attn(p, q=P, k=P, v=P, out=P):
    return lib.attn_chunk_fwd(q, k, v, out, None, ctypes.byref(p), None)


@pytest.mark.parametrize("kw,ptrs,status", [
    ({}, dict(q=None), skv.SKV_ERR_NULL),
    (dict(Hq=6, Hkv=4), {}, skv.SKV_ERR_SHAPE),
    (dict(Hq=16400, Hkv=2), {}, skv.SKV_ERR_SHAPE),  # Hq*D past 2^21 (32-bit row-block offsets)
    (dict(D=96), {}, skv.SKV_ERR_UNSUPPORTED),
    (dict(dtype=7), {}, skv.SKV_ERR_DTYPE),
    (dict(out_dtype=skv.SKV_F16), {}, skv.SKV_ERR_DTYPE),
    (dict(kv_len=0), {}, skv.SKV_ERR_RANGE),       # fish-speech #1312: 0 is invalid
    (dict(kv_len=65), {}, skv.SKV_ERR_RANGE),      # ... and so is capacity + 1
    (dict(mask=1, kv_len=4), {}, skv.SKV_ERR_RANGE),  # causal chunk longer than the prefix
    (dict(mask=2, mask_block=0), {}, skv.SKV_ERR_RANGE),
    (dict(mask=5), {}, skv.SKV_ERR_RANGE),
    (dict(flags=2), {}, skv.SKV_ERR_RANGE),
    (dict(scale=-1.0), {}, skv.SKV_ERR_RANGE),
    (dict(kv_len_dev=P, cu_seqlens_kv_dev=P), {}, skv.SKV_ERR_UNSUPPORTED),
    (dict(cu_seqlens_kv_dev=P, flags=skv.FULL_CAPACITY_MASKED), {}, skv.SKV_ERR_UNSUPPORTED),
    ({}, dict(k=BAD), skv.SKV_ERR_ALIGN),
    (dict(Tq=1), {}, skv.SKV_ERR_NULL),            # decode-sized call without a workspace
    (dict(Tq=1, workspace=P, workspace_bytes=16), {}, skv.SKV_ERR_RANGE),
])
def test_attention_host_errors(kw, ptrs, status):
    assert attn(params(**kw), **ptrs) == status
    assert lib.skv_last_error().decode()


def test_valid_kv_len_bounds_pass_validation_of_workspace_query():
    """1 and cap are valid (fish-speech #1312): the workspace query accepts them; decode-sized
    calls need a workspace, chunk-sized ones do not."""
    for kv_len in (1, 64):
        assert lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, kv_len=kv_len))) > 0
    assert lib.attn_workspace_bytes(ctypes.byref(params(Tq=8))) == 0
    # invalid parameters: a distinct result, never mistaken for "no workspace needed"
    invalid = ctypes.c_size_t(-1).value
    assert lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, kv_len=0))) == invalid
    assert "kv_len" in lib.skv_last_error().decode()
    assert lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, kv_len=65))) == invalid
    assert lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, D=96))) == invalid
    assert lib.attn_workspace_bytes(None) == invalid
    # the split-K workspace grows with the longest prefix it may see
    small = lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, kv_len=64, cap=64)))
    large = lib.attn_workspace_bytes(ctypes.byref(params(Tq=1, kv_len=4096, cap=4096)))
    assert large > small


def flash_tail_plan(B, Hq, Tq, key_bound):
    """The chunk-attention tail split restated: 64 resident workgroups per XCD; with I items
    per XCD, F whole rounds and R items left, cut those R into the k pieces (2..8, each piece
    at least 16 tiles of 64 keys at the bound) that minimise F + ceil(R k / 64) / k, if that
    saves 5% of the F + 1 rounds."""
    nq = -(-Tq // 128)
    if (B * Hq) % 8:
        return 1, 0
    I = nq * B * Hq // 8
    F, R = divmod(I, 64)
    if F == 0 or R == 0:
        return 1, 0
    best, bk = F + 1.0, 1
    for k in range(2, 9):
        if key_bound < k * 16 * 64:
            break
        cost = F + (-(-R * k // 64)) / k
        if cost < best - 1e-9:
            best, bk = cost, k
    return (bk, R) if bk > 1 and best <= 0.95 * (F + 1) else (1, 0)


@pytest.mark.parametrize("B,Hq,Tq,kv_len,D", [
    (2, 12, 4680, 32760, 128),   # ring: 37 query tiles x 24 heads, 111 items per XCD -> 4 pieces
    (2, 8, 4700, 6500, 128),     # 74 items per XCD, 10 left over -> 6 pieces
    (2, 8, 4700, 6500, 64),
    (2, 8, 4700, 5000, 128),     # bound allows 4 pieces only
    (2, 8, 4700, 1500, 128),     # pieces would be too short: no split
    (8, 40, 1024, 16384, 128),   # 320 items per XCD = 5 whole rounds: no split
    (2, 3, 4700, 6500, 128),     # heads do not divide over the XCDs: no split
    (1, 8, 4700, 6500, 128),     # 37 items per XCD, one round: no split
])
def test_flash_tail_split_workspace(B, Hq, Tq, kv_len, D):
    """attn_workspace_bytes of chunk-sized calls: zero unless the tail split is planned, then
    the shared 64 KiB counter area and one partial of 256 lanes x (D/2 + 2) floats per piece."""
    k, R = flash_tail_plan(B, Hq, Tq, kv_len)
    n_split = 8 * R
    want = 0 if k == 1 else 4 * (16384 + n_split * k * 256 * (D // 2 + 2))  # 64 KiB of counters first
    p = params(B=B, Hq=Hq, Hkv=Hq if Hq % 2 else Hq // 2, Tq=Tq, D=D, cap=kv_len, kv_len=kv_len)
    assert lib.attn_workspace_bytes(ctypes.byref(p)) == want
    if (B, Hq, Tq) == (2, 12, 4680):
        assert (k, R) == (4, 47)


def test_decode_workspace_layout_and_batch_limit():
    """Decode-sized calls: 64 KiB of counters, then o partials [B*Hkv*splits*16*D] and (m, l)
    [B*Hkv*splits*32] fp32; with B*Hkv >= 16384 they take the chunk path (no split-K
    workspace) and the fused step refuses them."""
    p = params(Tq=1, kv_len=4096, cap=4096, B=1, Hq=32, Hkv=8)
    splits = 32  # min(ceil(4096 / 128), 256 / 8)
    want = 4 * (16384 + 8 * splits * 16 * 128 + 8 * splits * 32)
    assert lib.attn_workspace_bytes(ctypes.byref(p)) == want
    big = params(Tq=1, kv_len=64, cap=64, B=2048, Hq=64, Hkv=8)  # B*Hkv = 16384
    assert lib.attn_workspace_bytes(ctypes.byref(big)) == 0
    f = lib.attn_decode_step
    # q, k_new, v_new, k_cache, v_cache, out, lse, cursor, kv_len_out, params, stream
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(big), None) == skv.SKV_ERR_UNSUPPORTED


def test_write_host_errors():
    f = lib.kv_write_indexed
    # k_cache, v_cache, k_src, v_src, index, start, B, cap, n, Hkv, D, dtype, err, stream
    assert f(None, None, P, None, None, 0, 1, 8, 1, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_NULL
    assert f(P, P, P, None, None, 0, 1, 8, 1, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_NULL
    assert f(P, None, P, None, None, 0, 1, 8, 1, 1, 64, 9, None, None) == skv.SKV_ERR_DTYPE
    assert f(P, None, P, None, None, 0, 1, 8, 1, 1, 3, skv.SKV_BF16, None, None) == skv.SKV_ERR_ALIGN
    assert f(BAD, None, P, None, None, 0, 1, 8, 1, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_ALIGN
    assert f(P, None, P, None, None, 5, 1, 8, 4, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_RANGE
    assert f(P, None, P, None, None, -1, 1, 8, 1, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_RANGE
    # empty writes are valid no-ops that launch nothing
    assert f(P, None, P, None, None, 0, 0, 8, 4, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_OK
    assert f(P, None, P, None, None, 0, 1, 8, 0, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_OK


def test_cursor_and_ring_host_errors():
    assert lib.kv_cursor_advance(None, 1, 8, 1, P, None, None, None) == skv.SKV_ERR_NULL
    assert lib.kv_cursor_advance(P, 0, 8, 1, P, None, None, None) == skv.SKV_ERR_SHAPE
    assert lib.kv_ring_meta_bytes(3) == 48
    h = ctypes.c_void_p()
    # 0 <= sink < n_slots (flashdreams #763: the sink is part of the window, at least one
    # rolling slot must remain)
    for n_slots, sink in ((4, 4), (4, -1), (0, 0)):
        st = lib.kv_ring_create(ctypes.byref(h), P, P, P, 2, 16, n_slots, sink, 1, 64, skv.SKV_BF16, None)
        assert st == skv.SKV_ERR_RANGE and not h.value
    st = lib.kv_ring_create(ctypes.byref(h), P, P, P, 2, 16, 4, 1, 1, 64, 11, None)
    assert st == skv.SKV_ERR_DTYPE
    assert lib.kv_ring_reserve(None, None, None) == skv.SKV_ERR_NULL
    assert lib.kv_ring_write(None, P, P, None, None, None) == skv.SKV_ERR_NULL
    assert lib.kv_ring_reset(None, None, None) == skv.SKV_ERR_NULL
    assert lib.kv_ring_kv_len_dev(None) is None


def test_decode_step_host_errors():
    f = lib.attn_decode_step
    p = params(Tq=1)
    assert f(P, None, P, P, P, P, None, P, None, ctypes.byref(p), None) == skv.SKV_ERR_NULL
    p = params(Tq=1, kv_len_dev=P)
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(p), None) == skv.SKV_ERR_UNSUPPORTED
    p = params(Tq=8)  # chunk-sized: not a decode step
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(p), None) == skv.SKV_ERR_UNSUPPORTED
    p = params(Tq=1, dtype=skv.SKV_F32, out_dtype=skv.SKV_F32)
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(p), None) == skv.SKV_ERR_UNSUPPORTED
    p = params(Tq=1)
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(p), None) == skv.SKV_ERR_NULL  # workspace


def test_roll_and_pack_host_errors():
    f = lib.kv_roll_left
    # k_store, v_store, B, rows, sink_rows, shift_rows, Hkv, D, dtype, stream
    assert f(None, None, 1, 8, 1, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_ERR_NULL
    assert f(P, None, 1, 8, 1, 2, 1, 64, 9, None) == skv.SKV_ERR_DTYPE
    assert f(P, None, 1, 8, 7, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_ERR_RANGE  # sink+shift > rows
    assert f(P, None, 1, 8, -1, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_ERR_RANGE
    assert f(P, None, 1, 8, 1, 0, 1, 64, skv.SKV_BF16, None) == skv.SKV_ERR_RANGE
    assert f(BAD, None, 1, 8, 1, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_ERR_ALIGN
    assert f(P, None, 1, 8, 1, 2, 1, 3, skv.SKV_BF16, None) == skv.SKV_ERR_ALIGN  # 6-byte rows
    assert f(P, None, 1, 8, 6, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_OK      # nothing to move
    assert f(P, None, 0, 8, 1, 2, 1, 64, skv.SKV_BF16, None) == skv.SKV_OK      # B = 0
    g = lib.kv_ragged_metadata
    assert g(None, 2, 8, P, None, None) == skv.SKV_ERR_NULL
    assert g(P, 0, 8, P, None, None) == skv.SKV_ERR_SHAPE
    assert g(P + 2, 2, 8, P, None, None) == skv.SKV_ERR_ALIGN
    h = lib.kv_pack_ragged
    # k_packed, v_packed, k_padded, v_padded, cu, B, max_kv, packed_rows, Hkv, D, dtype, err, stream
    assert h(P, None, P, None, None, 2, 8, 16, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_NULL
    assert h(P, P, P, None, P, 2, 8, 16, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_NULL
    assert h(P, None, P, None, P, 2, 8, 16, 1, 64, 5, None, None) == skv.SKV_ERR_DTYPE
    assert h(P, None, P, None, P, 0, 8, 16, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_SHAPE
    assert h(BAD, None, P, None, P, 2, 8, 16, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_ERR_ALIGN
    assert h(P, None, P, None, P, 2, 0, 16, 1, 64, skv.SKV_BF16, None, None) == skv.SKV_OK  # nothing


def test_rope_write_host_errors():
    f = lib.kv_write_indexed_rope
    # k_cache, v_cache, k_src, v_src, index, start, B, cap, n, Hkv, D, dtype, inv_freq, layout, err, stream
    ok = (P, None, P, None, None, 0, 1, 64, 8, 2, 128, skv.SKV_BF16, P, skv.ROPE_HALF, None, None)
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[["kc", "vc", "ks", "vs", "idx", "start", "B", "cap", "n", "Hkv", "D", "dt", "freq",
               "layout", "err", "st"].index(k)] = v
        return f(*a)
    assert call(freq=None) == skv.SKV_ERR_NULL
    assert call(freq=P + 4) == skv.SKV_ERR_ALIGN
    assert call(layout=2) == skv.SKV_ERR_RANGE
    assert call(D=96) == skv.SKV_ERR_SHAPE      # not a power of two
    assert call(D=8) == skv.SKV_ERR_SHAPE       # fewer than 8 pairs
    assert call(dt=7) == skv.SKV_ERR_DTYPE
    assert call(kc=None) == skv.SKV_ERR_NULL
    assert call(vc=P) == skv.SKV_ERR_NULL       # V cache without V source
    assert call(start=60) == skv.SKV_ERR_RANGE  # rows 60..67 past cap 64
    assert call(kc=BAD) == skv.SKV_ERR_ALIGN
    assert call(B=0) == skv.SKV_OK and call(n=0) == skv.SKV_OK
    g = lib.kv_ring_write_rope
    # ring, k_src, v_src, inv_freq, layout, mask, err, stream
    assert g(None, P, None, P, 0, None, None, None) == skv.SKV_ERR_NULL


def test_probe_host_errors():
    f, c = lib.skv_probe_mfma_bf16, lib.skv_probe_copy
    assert f(None, 1, 1, None) == skv.SKV_ERR_NULL
    assert f(P, 0, 1, None) == skv.SKV_ERR_RANGE
    assert f(P, 1, 0, None) == skv.SKV_ERR_RANGE
    assert f(P + 2, 1, 1, None) == skv.SKV_ERR_ALIGN
    assert c(None, P, 16, None) == skv.SKV_ERR_NULL
    assert c(P, P, 24, None) == skv.SKV_ERR_SHAPE
    assert c(BAD, P, 16, None) == skv.SKV_ERR_ALIGN
    assert c(P, P, 0, None) == skv.SKV_OK  # nothing to do, nothing launched


def test_static_scratch_decode_step_host_errors():
    """attn_decode_step_static refuses, before touching the GPU, a step whose split-K scratch
    would not fit the static array, and shares the fused step's other host checks."""
    f = lib.attn_decode_step_static
    # q, k_new, v_new, k_cache, v_cache, out, lse, cursor, kv_len_out, params, stream
    big = params(Tq=1, kv_len=32768, cap=32768, B=64, Hq=64, Hkv=8)
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(big), None) == skv.SKV_ERR_RANGE
    assert "static scratch" in lib.skv_last_error().decode()
    assert f(P, None, P, P, P, P, None, P, None, ctypes.byref(big), None) == skv.SKV_ERR_NULL
    packed = params(Tq=1, kv_len=64, cap=64, cu_seqlens_kv_dev=P)
    assert f(P, P, P, P, P, P, None, P, None, ctypes.byref(packed), None) == skv.SKV_ERR_UNSUPPORTED
