"""MI355X-native chunk attention over a preallocated KV cache.

The product is libskv.so (C ABI in include/skv.h, HIP kernels for gfx950 in csrc/); this
package is its thin Python binding. Build with `python streaming_kv_cache_write_amd/build.py`.
Importing fails loudly if the library is not built: there is no fallback path.
"""
from ._binding import (  # noqa: F401
    DEV_CU_SEQLENS, DEV_CURSOR_FULL, DEV_INDEX_RANGE, DEV_KV_LEN, DEV_RING_UNRESERVED, EXPORTED,
    FULL_CAPACITY_MASKED, LIB_PATH, MASK_BLOCK_CAUSAL, MASK_CAUSAL, MASK_NONE, ROPE_HALF,
    ROPE_INTERLEAVED, SKV_BF16,
    SKV_ERR_ALIGN, SKV_ERR_DTYPE, SKV_ERR_HIP, SKV_ERR_NULL, SKV_ERR_RANGE, SKV_ERR_SHAPE,
    SKV_ERR_UNSUPPORTED, SKV_F16, SKV_F32, SKV_OK, Ring, SkvError, attn_chunk_fwd, attn_decode_step,
    attn_workspace_bytes, kv_cursor_advance, kv_pack_ragged, kv_ragged_metadata, kv_roll_left,
    kv_write_indexed, kv_write_indexed_rope, lib, make_params, probe_copy, probe_mfma_bf16,
    skv_attn_params)
