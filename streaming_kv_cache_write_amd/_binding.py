"""ctypes binding of libskv (include/skv.h): argument marshalling only.

Every function here takes torch tensors, checks that they are contiguous device tensors of
the right dtype, derives the sizes the C call needs, and calls the C entry point of the same
name on torch's current HIP stream. All arithmetic runs in the library's HIP kernels; there
is no fallback of any kind: if libskv.so is missing this module fails to import.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SKV_LIBRARY names another build of the same library: the CPU ABI tests load the host-side
# AddressSanitizer build through it; it is never a fallback.
LIB_PATH = os.environ.get("SKV_LIBRARY") or os.path.join(_HERE, "libskv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python streaming_kv_cache_write_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------------------ constants
SKV_OK, SKV_ERR_NULL, SKV_ERR_SHAPE, SKV_ERR_RANGE, SKV_ERR_DTYPE, SKV_ERR_ALIGN, \
    SKV_ERR_UNSUPPORTED, SKV_ERR_HIP = range(8)
STATUS_NAMES = ["SKV_OK", "SKV_ERR_NULL", "SKV_ERR_SHAPE", "SKV_ERR_RANGE", "SKV_ERR_DTYPE",
                "SKV_ERR_ALIGN", "SKV_ERR_UNSUPPORTED", "SKV_ERR_HIP"]
SKV_F32, SKV_F16, SKV_BF16 = 0, 1, 2
MASK_NONE, MASK_CAUSAL, MASK_BLOCK_CAUSAL = 0, 1, 2
ROPE_HALF, ROPE_INTERLEAVED = 0, 1  # pair (i, i + D/2) or (2i, 2i + 1)
FULL_CAPACITY_MASKED = 1
DEV_INDEX_RANGE, DEV_KV_LEN, DEV_CU_SEQLENS, DEV_RING_UNRESERVED, DEV_CURSOR_FULL = 1, 2, 4, 8, 16

_DTYPES = {torch.float32: SKV_F32, torch.float16: SKV_F16, torch.bfloat16: SKV_BF16}


class SkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


class skv_attn_params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("Tq", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
        ("D", ctypes.c_int),
        ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("cap", ctypes.c_int), ("kv_len", ctypes.c_int),
        ("kv_len_dev", ctypes.c_void_p), ("cu_seqlens_kv_dev", ctypes.c_void_p),
        ("max_seqlen_kv", ctypes.c_int),
        ("mask", ctypes.c_int), ("mask_block", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("err_dev", ctypes.c_void_p),
    ]


_vp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "skv_last_error": (ctypes.c_char_p, []),
    "skv_version": (ctypes.c_char_p, []),
    "kv_write_indexed": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "kv_write_indexed_rope": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i, _i, _i, _i, _i, _i, _vp, _i,
                                   _vp, _vp]),
    "kv_cursor_advance": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "kv_ring_meta_bytes": (_sz, [_i]),
    "kv_ring_create": (_i, [ctypes.POINTER(_vp), _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "kv_ring_reserve": (_i, [_vp, _vp, _vp]),
    "kv_ring_write": (_i, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "kv_ring_write_rope": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "kv_ring_reset": (_i, [_vp, _vp, _vp]),
    "kv_ring_kv_len_dev": (_vp, [_vp]),
    "kv_ring_slot_dev": (_vp, [_vp]),
    "kv_ring_destroy": (_i, [_vp]),
    "kv_roll_left": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "kv_ragged_metadata": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "kv_pack_ragged": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "attn_workspace_bytes": (_sz, [ctypes.POINTER(skv_attn_params)]),
    "attn_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, ctypes.POINTER(skv_attn_params), _vp]),
    "attn_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              ctypes.POINTER(skv_attn_params), _vp]),
    "attn_decode_step_static": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(skv_attn_params), _vp]),
    "skv_probe_mfma_bf16": (_i, [_vp, _i, _i, _vp]),
    "skv_probe_copy": (_i, [_vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args
EXPORTED = tuple(_SIGS)


def _check(status: int) -> None:
    if status != SKV_OK:
        raise SkvError(status, lib.skv_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _shape(t, shape, name: str):
    """Shape check before any C call: the C ABI takes raw pointers, so a tensor whose size does
    not match the sizes passed with it would be read or written out of bounds on the device."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ndim(t, n: int, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions (got shape {tuple(t.shape)})")
    return t.shape


def _numel(t, n: int, name: str, at_least: bool = False):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if (t.numel() < n) if at_least else (t.numel() != n):
        raise ValueError(f"{name} has {t.numel()} elements, expected {'at least ' if at_least else ''}{n}")
    return t


# One zero-filled workspace per (device, stream), grown on demand, for calls that do not bring
# their own: calls on one stream are ordered, and each leaves the workspace's arrival counters
# at zero for the next. Calls recorded into a HIP graph get a fresh one (allocated from the
# graph's pool); callers that replay graphs or run concurrent streams pass their own.
_WORKSPACES: dict = {}


def _workspace(device, need: int):
    if need <= 0:
        return None
    if torch.cuda.is_current_stream_capturing():
        return torch.zeros(need, dtype=torch.uint8, device=device)
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _DTYPES[dtype]


# ------------------------------------------------------------------------------ writes
def kv_write_indexed(k_cache, v_cache, k_src, v_src, index=None, start: int = 0, err=None):
    """k_cache[b, index[t]] = k_src[b, t] (and V); index None -> rows start .. start+n."""
    B, cap, Hkv, D = _ndim(k_cache, 4, "k_cache")
    n = _ndim(k_src, 4, "k_src")[1]
    _shape(k_src, (B, n, Hkv, D), "k_src")
    _shape(v_cache, k_cache.shape, "v_cache")
    _shape(v_src, k_src.shape, "v_src")
    _numel(index, n, "index")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(k_cache, "k_cache")
    _dev_tensor(k_src, "k_src", k_cache.dtype)
    if v_cache is not None:
        _dev_tensor(v_cache, "v_cache", k_cache.dtype)
        _dev_tensor(v_src, "v_src", k_cache.dtype)
    if index is not None:
        _dev_tensor(index, "index", torch.int64)
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    n = k_src.shape[1]
    _check(lib.kv_write_indexed(_ptr(k_cache), _ptr(v_cache), _ptr(k_src), _ptr(v_src), _ptr(index),
                                int(start), B, cap, n, Hkv, D, dtype_code(k_cache.dtype), _ptr(err),
                                _stream(k_cache.device)))


def _inv_freq(inv_freq, D: int):
    _dev_tensor(inv_freq, "inv_freq", torch.float64)
    if inv_freq.numel() != D // 2:
        raise ValueError(f"inv_freq must hold D/2 = {D // 2} frequencies (got {inv_freq.numel()})")
    return inv_freq


def kv_write_indexed_rope(k_cache, v_cache, k_src, v_src, inv_freq, rope_layout: int = ROPE_HALF,
                          index=None, start: int = 0, err=None):
    """kv_write_indexed with K rotated at its destination row: inv_freq float64 [D/2] on the
    device, rope_layout ROPE_HALF or ROPE_INTERLEAVED."""
    B, cap, Hkv, D = _ndim(k_cache, 4, "k_cache")
    n = _ndim(k_src, 4, "k_src")[1]
    _shape(k_src, (B, n, Hkv, D), "k_src")
    _shape(v_cache, k_cache.shape, "v_cache")
    _shape(v_src, k_src.shape, "v_src")
    _numel(index, n, "index")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(k_cache, "k_cache")
    _dev_tensor(k_src, "k_src", k_cache.dtype)
    if v_cache is not None:
        _dev_tensor(v_cache, "v_cache", k_cache.dtype)
        _dev_tensor(v_src, "v_src", k_cache.dtype)
    if index is not None:
        _dev_tensor(index, "index", torch.int64)
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    _inv_freq(inv_freq, D)
    n = k_src.shape[1]
    _check(lib.kv_write_indexed_rope(_ptr(k_cache), _ptr(v_cache), _ptr(k_src), _ptr(v_src),
                                     _ptr(index), int(start), B, cap, n, Hkv, D,
                                     dtype_code(k_cache.dtype), _ptr(inv_freq), int(rope_layout),
                                     _ptr(err), _stream(k_cache.device)))


def kv_cursor_advance(cursor, n: int, cap: int, index_out, kv_len_out=None, err=None):
    """index_out[t] = cursor + t, kv_len_out[:] = cursor + n, cursor += n, all on the device."""
    _numel(cursor, 1, "cursor", at_least=True)
    _numel(index_out, int(n), "index_out")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(cursor, "cursor", torch.int32)
    _dev_tensor(index_out, "index_out", torch.int64)
    B = 0
    if kv_len_out is not None:
        _dev_tensor(kv_len_out, "kv_len_out", torch.int32)
        B = kv_len_out.numel()
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    _check(lib.kv_cursor_advance(_ptr(cursor), int(n), int(cap), B, _ptr(index_out),
                                 _ptr(kv_len_out), _ptr(err), _stream(cursor.device)))


def kv_roll_left(k_store, v_store, sink_rows: int, shift_rows: int):
    """Move rows [sink_rows + shift_rows, rows) of k_store/v_store [B, rows, Hkv, D] to
    [sink_rows, rows - shift_rows) (memmove semantics): the chronological window's roll-left."""
    B, rows, Hkv, D = _ndim(k_store, 4, "k_store")
    _shape(v_store, k_store.shape, "v_store")
    _dev_tensor(k_store, "k_store")
    if v_store is not None:
        _dev_tensor(v_store, "v_store", k_store.dtype)
    _check(lib.kv_roll_left(_ptr(k_store), _ptr(v_store), B, rows, int(sink_rows), int(shift_rows),
                            Hkv, D, dtype_code(k_store.dtype), _stream(k_store.device)))


def kv_ragged_metadata(lens, max_kv: int, cu_seqlens_out=None, err=None):
    """cu_seqlens_kv [B+1] int32 (exclusive prefix sums of lens [B] int32), on the device."""
    B = lens.numel()
    _numel(cu_seqlens_out, B + 1, "cu_seqlens_out")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(lens, "lens", torch.int32)
    if cu_seqlens_out is None:
        cu_seqlens_out = torch.empty(B + 1, dtype=torch.int32, device=lens.device)
    _dev_tensor(cu_seqlens_out, "cu_seqlens_out", torch.int32)
    if cu_seqlens_out.numel() != B + 1:
        raise ValueError("cu_seqlens_out must have B+1 entries")
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    _check(lib.kv_ragged_metadata(_ptr(lens), B, int(max_kv), _ptr(cu_seqlens_out), _ptr(err),
                                  _stream(lens.device)))
    return cu_seqlens_out


def kv_pack_ragged(k_padded, v_padded, cu_seqlens, k_packed, v_packed=None, err=None):
    """Rows [0, len_b) of k_padded/v_padded [B, max_kv, Hkv, D] to rows [cu[b], cu[b+1]) of
    k_packed/v_packed [packed_rows, Hkv, D], len_b = cu[b+1] - cu[b]."""
    B, max_kv, Hkv, D = _ndim(k_padded, 4, "k_padded")
    _shape(v_padded, k_padded.shape, "v_padded")
    _shape(k_packed, (_ndim(k_packed, 3, "k_packed")[0], Hkv, D), "k_packed")
    _shape(v_packed, k_packed.shape, "v_packed")
    _numel(cu_seqlens, B + 1, "cu_seqlens")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(k_padded, "k_padded")
    _dev_tensor(k_packed, "k_packed", k_padded.dtype)
    if v_padded is not None:
        _dev_tensor(v_padded, "v_padded", k_padded.dtype)
        _dev_tensor(v_packed, "v_packed", k_padded.dtype)
    _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32)
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    _check(lib.kv_pack_ragged(_ptr(k_packed), _ptr(v_packed), _ptr(k_padded), _ptr(v_padded),
                              _ptr(cu_seqlens), B, max_kv, k_packed.shape[0], Hkv, D,
                              dtype_code(k_padded.dtype), _ptr(err), _stream(k_padded.device)))


class Ring:
    """Sink-plus-window ring over caller storage k_store/v_store [B, n_slots*chunk, Hkv, D]."""

    def __init__(self, k_store, v_store, chunk: int, n_slots: int, sink_slots: int, meta=None):
        B, rows, Hkv, D = _ndim(k_store, 4, "k_store")
        _shape(v_store, k_store.shape, "v_store")
        _dev_tensor(k_store, "k_store")
        if rows != n_slots * chunk:
            raise ValueError(f"storage has {rows} rows, expected n_slots*chunk = {n_slots * chunk}")
        if v_store is not None:
            _dev_tensor(v_store, "v_store", k_store.dtype)
        nbytes = lib.kv_ring_meta_bytes(B)
        if meta is None:
            meta = torch.empty(nbytes // 4, dtype=torch.int32, device=k_store.device)
        _dev_tensor(meta, "meta", torch.int32)
        if meta.numel() * 4 < nbytes:
            raise ValueError("meta buffer too small")
        self.k_store, self.v_store, self.meta = k_store, v_store, meta
        self.B, self.chunk, self.n_slots, self.sink = B, chunk, n_slots, sink_slots
        self._h = ctypes.c_void_p()
        _check(lib.kv_ring_create(ctypes.byref(self._h), _ptr(k_store), _ptr(v_store), _ptr(meta),
                                  B, chunk, n_slots, sink_slots, Hkv, D, dtype_code(k_store.dtype),
                                  _stream(k_store.device)))

    @property
    def handle(self) -> int:
        return self._h.value

    def reserve(self, batch_mask=None):
        _numel(batch_mask, self.B, "batch_mask")
        if batch_mask is not None:
            _dev_tensor(batch_mask, "batch_mask", torch.uint8)
        _check(lib.kv_ring_reserve(self._h, _ptr(batch_mask), _stream(self.k_store.device)))

    def _check_sources(self, k_src, v_src, batch_mask, err):
        _, _, Hkv, D = self.k_store.shape
        _shape(k_src, (self.B, self.chunk, Hkv, D), "k_src")
        _shape(v_src, k_src.shape, "v_src")
        _numel(batch_mask, self.B, "batch_mask")
        _numel(err, 1, "err", at_least=True)

    def write(self, k_src, v_src=None, batch_mask=None, err=None):
        self._check_sources(k_src, v_src, batch_mask, err)
        _dev_tensor(k_src, "k_src", self.k_store.dtype)
        if v_src is not None:
            _dev_tensor(v_src, "v_src", self.k_store.dtype)
        if batch_mask is not None:
            _dev_tensor(batch_mask, "batch_mask", torch.uint8)
        if err is not None:
            _dev_tensor(err, "err", torch.int32)
        if k_src.shape[0] != self.B or k_src.shape[1] != self.chunk:
            raise ValueError(f"source must be [B={self.B}, chunk={self.chunk}, Hkv, D]")
        _check(lib.kv_ring_write(self._h, _ptr(k_src), _ptr(v_src), _ptr(batch_mask), _ptr(err),
                                 _stream(self.k_store.device)))

    def write_rope(self, k_src, v_src, inv_freq, rope_layout: int = ROPE_HALF, batch_mask=None,
                   err=None):
        """write() with K rotated at chunk_id * chunk + t (chunk_id since the last reset)."""
        self._check_sources(k_src, v_src, batch_mask, err)
        _dev_tensor(k_src, "k_src", self.k_store.dtype)
        if v_src is not None:
            _dev_tensor(v_src, "v_src", self.k_store.dtype)
        if batch_mask is not None:
            _dev_tensor(batch_mask, "batch_mask", torch.uint8)
        if err is not None:
            _dev_tensor(err, "err", torch.int32)
        if k_src.shape[0] != self.B or k_src.shape[1] != self.chunk:
            raise ValueError(f"source must be [B={self.B}, chunk={self.chunk}, Hkv, D]")
        _inv_freq(inv_freq, self.k_store.shape[3])
        _check(lib.kv_ring_write_rope(self._h, _ptr(k_src), _ptr(v_src), _ptr(inv_freq),
                                      int(rope_layout), _ptr(batch_mask), _ptr(err),
                                      _stream(self.k_store.device)))

    def reset(self, batch_mask=None):
        _numel(batch_mask, self.B, "batch_mask")
        if batch_mask is not None:
            _dev_tensor(batch_mask, "batch_mask", torch.uint8)
        _check(lib.kv_ring_reset(self._h, _ptr(batch_mask), _stream(self.k_store.device)))

    @property
    def kv_len(self):
        """[B] int32 device view of the retained-token counts (attention's kv_len_dev)."""
        return self.meta[3 * self.B:4 * self.B]

    @property
    def slot(self):
        return self.meta[self.B:2 * self.B]

    @property
    def counter(self):
        return self.meta[:self.B]

    def close(self):
        if self._h:
            lib.kv_ring_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------ attention
def make_params(q, k, *, kv_len=None, kv_len_dev=None, cu_seqlens_kv=None, max_seqlen_kv=0,
                mask=MASK_NONE, mask_block=1, scale=0.0, full_capacity_masked=False,
                out_dtype=None, workspace=None, err=None) -> skv_attn_params:
    B, Tq, Hq, D = q.shape
    if cu_seqlens_kv is not None:
        cap, Hkv = k.shape[0], k.shape[1]
    else:
        if k.shape[0] != B:
            raise ValueError(f"k has batch {k.shape[0]}, q has {B}")
        cap, Hkv = k.shape[1], k.shape[2]
    p = skv_attn_params()
    p.B, p.Tq, p.Hq, p.Hkv, p.D = B, Tq, Hq, Hkv, D
    p.dtype = dtype_code(q.dtype)
    p.out_dtype = dtype_code(out_dtype) if out_dtype is not None else p.dtype
    p.cap = cap
    p.kv_len = int(kv_len) if kv_len is not None else 0
    p.kv_len_dev = _ptr(kv_len_dev)
    p.cu_seqlens_kv_dev = _ptr(cu_seqlens_kv)
    p.max_seqlen_kv = int(max_seqlen_kv)
    p.mask, p.mask_block = int(mask), int(mask_block)
    p.scale = float(scale)
    p.flags = FULL_CAPACITY_MASKED if full_capacity_masked else 0
    p.workspace = _ptr(workspace)
    p.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    p.err_dev = _ptr(err)
    return p


SIZE_INVALID = ctypes.c_size_t(-1).value  # attn_workspace_bytes of an invalid parameter set


def _workspace_need(q, k, **kw) -> int:
    """Workspace bytes for these parameters, or 0 if they are invalid (the call itself then
    returns the precise status)."""
    n = int(lib.attn_workspace_bytes(ctypes.byref(make_params(q, k, **kw))))
    return 0 if n == SIZE_INVALID else n


def attn_workspace_bytes(q, k, **kw) -> int:
    """Workspace bytes a call with these arguments needs; ValueError if they are invalid."""
    n = int(lib.attn_workspace_bytes(ctypes.byref(make_params(q, k, **kw))))
    if n == SIZE_INVALID:
        raise ValueError(f"invalid attention parameters: {lib.skv_last_error().decode()}")
    return n


def _check_attn_shapes(q, k, v, out, lse, kv_len_dev, cu_seqlens_kv, err):
    B, Tq, Hq, D = _ndim(q, 4, "q")
    if cu_seqlens_kv is not None and kv_len_dev is not None:
        return  # an unsupported combination: the library refuses it before any launch
    if cu_seqlens_kv is not None:
        _shape(k, (_ndim(k, 3, "k")[0], k.shape[1], D), "k")
        _numel(cu_seqlens_kv, B + 1, "cu_seqlens_kv")
    else:
        _shape(k, (B, _ndim(k, 4, "k")[1], k.shape[2], D), "k")
    _shape(v, k.shape, "v")
    _shape(out, q.shape, "out")
    _shape(lse, (B, Hq, Tq), "lse")
    _numel(kv_len_dev, B, "kv_len_dev")
    _numel(err, 1, "err", at_least=True)


def attn_chunk_fwd(q, k, v, out=None, lse=None, *, kv_len=None, kv_len_dev=None,
                   cu_seqlens_kv=None, max_seqlen_kv=0, mask=MASK_NONE, mask_block=1, scale=0.0,
                   full_capacity_masked=False, out_dtype=None, workspace=None, err=None):
    """Attention of q [B, Tq, Hq, D] over k/v [B, cap, Hkv, D] (prefix: host kv_len or device
    kv_len_dev [B] int32) or packed k/v [total, Hkv, D] (cu_seqlens_kv [B+1] int32).
    Returns out [B, Tq, Hq, D] (and fills lse [B, Hq, Tq] fp32 if given). Without a workspace
    the call uses the one cached for its device and stream (see _workspace)."""
    _check_attn_shapes(q, k, v, out, lse, kv_len_dev, cu_seqlens_kv, err)
    _dev_tensor(q, "q")
    _dev_tensor(k, "k", q.dtype)
    _dev_tensor(v, "v", q.dtype)
    if kv_len_dev is not None:
        _dev_tensor(kv_len_dev, "kv_len_dev", torch.int32)
    if cu_seqlens_kv is not None:
        _dev_tensor(cu_seqlens_kv, "cu_seqlens_kv", torch.int32)
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    odt = out_dtype if out_dtype is not None else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    _dev_tensor(out, "out", odt)
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32)
    kw = dict(kv_len=kv_len, kv_len_dev=kv_len_dev, cu_seqlens_kv=cu_seqlens_kv,
              max_seqlen_kv=max_seqlen_kv, mask=mask, mask_block=mask_block, scale=scale,
              full_capacity_masked=full_capacity_masked, out_dtype=odt, err=err)
    if workspace is None:
        workspace = _workspace(q.device, _workspace_need(q, k, **kw))
    if workspace is not None:
        _dev_tensor(workspace, "workspace")
    p = make_params(q, k, workspace=workspace, **kw)
    _check(lib.attn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), ctypes.byref(p),
                              _stream(q.device)))
    return out


def attn_decode_step(q, k_new, v_new, k_cache, v_cache, cursor, out=None, lse=None, *,
                     kv_len_out=None, max_seqlen_kv=0, mask=MASK_NONE, mask_block=1, scale=0.0,
                     out_dtype=None, workspace=None, err=None, static_scratch=False):
    """One fused decode step: write k_new/v_new [B, Tq, Hkv, D] at the device cursor, attend q
    [B, Tq, Hq, D] over the cache prefix including them, advance the cursor (and fill
    kv_len_out [B]). Returns out. Without a workspace the call uses the cached one;
    static_scratch=True calls attn_decode_step_static instead (no workspace at all; out must
    then be given for the call to allocate nothing)."""
    B, Tq, Hq, D = _ndim(q, 4, "q")
    _, cap, Hkv, _ = _ndim(k_cache, 4, "k_cache")
    _shape(k_cache, (B, cap, Hkv, D), "k_cache")
    _shape(v_cache, k_cache.shape, "v_cache")
    _shape(k_new, (B, Tq, Hkv, D), "k_new")
    _shape(v_new, (B, Tq, Hkv, D), "v_new")
    _shape(out, q.shape, "out")
    _shape(lse, (B, Hq, Tq), "lse")
    _numel(cursor, 1, "cursor", at_least=True)
    _numel(kv_len_out, B, "kv_len_out")
    _numel(err, 1, "err", at_least=True)
    _dev_tensor(q, "q")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, q.dtype)
    _dev_tensor(cursor, "cursor", torch.int32)
    if kv_len_out is not None:
        _dev_tensor(kv_len_out, "kv_len_out", torch.int32)
    if err is not None:
        _dev_tensor(err, "err", torch.int32)
    odt = out_dtype if out_dtype is not None else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    _dev_tensor(out, "out", odt)
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32)
    bound = int(max_seqlen_kv) if max_seqlen_kv else cap
    kw = dict(max_seqlen_kv=max_seqlen_kv, mask=mask, mask_block=mask_block, scale=scale,
              out_dtype=odt, err=err)
    if static_scratch:
        p = make_params(q, k_cache, **kw)
        _check(lib.attn_decode_step_static(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(cursor),
                                           _ptr(kv_len_out), ctypes.byref(p), _stream(q.device)))
        return out
    if workspace is None:
        need = _workspace_need(q, k_cache, kv_len=max(min(bound, cap), Tq), **kw)
        workspace = _workspace(q.device, max(need, 16))
    _dev_tensor(workspace, "workspace")
    p = make_params(q, k_cache, workspace=workspace, **kw)
    _check(lib.attn_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(out), _ptr(lse), _ptr(cursor), _ptr(kv_len_out), ctypes.byref(p),
                                _stream(q.device)))
    return out


# ------------------------------------------------------------------------------ measurement
def probe_mfma_bf16(out, workgroups: int, iters: int) -> int:
    """Launch the back-to-back bf16 MFMA probe; out: fp32 device tensor of workgroups*256.
    Returns the flops it executes."""
    _dev_tensor(out, "out", torch.float32)
    if out.numel() < workgroups * 256:
        raise ValueError("out needs workgroups * 256 floats")
    _check(lib.skv_probe_mfma_bf16(_ptr(out), int(workgroups), int(iters), _stream(out.device)))
    return int(workgroups) * 16 * int(iters) * 32768


def probe_copy(dst, src) -> int:
    """Copy src to dst (device tensors of equal byte size) with the probe copy kernel.
    Returns the bytes of traffic (read + write)."""
    _dev_tensor(dst, "dst")
    _dev_tensor(src, "src")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("dst and src differ in size")
    _check(lib.skv_probe_copy(_ptr(dst), _ptr(src), nb, _stream(src.device)))
    return 2 * nb
