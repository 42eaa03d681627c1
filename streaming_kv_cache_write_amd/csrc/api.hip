// Host side of the libskv C ABI: argument validation, dispatch, launches on the caller's
// stream. Nothing here allocates device memory, synchronizes, or reads device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <string>

#include "common.h"

namespace skv {
hipError_t launch_write_indexed(const void*, const void*, void*, void*, const int64_t*, int64_t, int,
                                int, int, int, int32_t*, hipStream_t);
hipError_t launch_cursor_advance(int32_t*, int, int, int, int64_t*, int32_t*, int32_t*, hipStream_t);
hipError_t launch_ring_reset(int32_t*, int, const uint8_t*, hipStream_t);
hipError_t launch_ring_reserve(int32_t*, int, const uint8_t*, int, int, hipStream_t);
hipError_t launch_ring_write(const void*, const void*, void*, void*, int32_t*, int, const uint8_t*,
                             int, int, int, int32_t*, hipStream_t);
hipError_t launch_roll_left(void*, void*, int, int, int, int, int, hipStream_t);
hipError_t launch_ragged_metadata(const int32_t*, int, int, int32_t*, int32_t*, hipStream_t);
hipError_t launch_pack_ragged(const void*, const void*, void*, void*, const int32_t*, int, int, int,
                              int, int32_t*, hipStream_t);
hipError_t launch_write_indexed_rope(const void*, const void*, void*, void*, const int64_t*, int64_t,
                                     int, int, int, int, int, int, const double*, int, int32_t*,
                                     hipStream_t);
hipError_t launch_ring_write_rope(const void*, const void*, void*, void*, int32_t*, int,
                                  const uint8_t*, int, int, int, int, int, const double*, int,
                                  int32_t*, hipStream_t);
hipError_t launch_attn_f32(const AttnArgs&, int, hipStream_t);
hipError_t launch_peak_mfma_bf16(float*, int, int, hipStream_t);
hipError_t launch_peak_copy(void*, const void*, size_t, hipStream_t);
hipError_t launch_attn_flash(const AttnArgs&, int, int, int, int, void*, size_t, hipStream_t);
size_t flash_workspace_bytes(int B, int Hq, int Tq, int D, int key_bound);
hipError_t launch_attn_decode(const AttnArgs&, int, int, int, void*, int, int, hipStream_t);
int decode_splits(int B, int Hkv, int max_len);
size_t decode_workspace_bytes(int B, int Hkv, int D, int n_splits);
}  // namespace skv

using namespace skv;

namespace {

thread_local std::string g_err;

skv_status fail(skv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

skv_status ok() {
  g_err.clear();
  return SKV_OK;
}

skv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case SKV_F32: return 4;
    case SKV_F16: return 2;
    case SKV_BF16: return 2;
    default: return 0;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kDecodeMaxTq = 4;
constexpr int kDecodeMaxRows = 16;

// Path taken by attn_chunk_fwd for a validated parameter set.
enum Path { PATH_F32, PATH_FLASH, PATH_DECODE };

// (the split-K path counts arrivals per (b, KV head) in the workspace's shared counter area,
// so it takes B*Hkv below its size; larger batches of short chunks run the flash path)
Path choose_path(const skv_attn_params& p) {
  if (p.dtype == SKV_F32) return PATH_F32;
  if (p.Tq <= kDecodeMaxTq && p.Tq * (p.Hq / p.Hkv) <= kDecodeMaxRows &&
      (int64_t)p.B * p.Hkv < kWsCounterInts)
    return PATH_DECODE;
  return PATH_FLASH;
}

// Host bound on the keys any batch element attends to (sizes split grids and workspaces).
int key_bound(const skv_attn_params& p) {
  if (p.flags & SKV_FULL_CAPACITY_MASKED) return p.cap;
  if (p.cu_seqlens_kv_dev || p.kv_len_dev)
    return p.max_seqlen_kv > 0 ? (p.max_seqlen_kv < p.cap ? p.max_seqlen_kv : p.cap) : p.cap;
  return p.kv_len;
}

skv_status validate_attn(const void* q, const void* k, const void* v, const void* out,
                         const skv_attn_params* p) {
  if (!p) return fail(SKV_ERR_NULL, "params is NULL");
  if (!q || !k || !v || !out) return fail(SKV_ERR_NULL, "q, k, v and out must be non-NULL");
  const bool packed = p->cu_seqlens_kv_dev != nullptr;
  if (packed && p->kv_len_dev)
    return fail(SKV_ERR_UNSUPPORTED, "kv_len_dev and cu_seqlens_kv_dev are exclusive");
  if (packed && (p->flags & SKV_FULL_CAPACITY_MASKED))
    return fail(SKV_ERR_UNSUPPORTED, "the full-capacity arm needs prefix (slab) mode");
  if (p->B < 1 || p->Tq < 0 || p->Hq < 1 || p->Hkv < 1)
    return fail(SKV_ERR_SHAPE, "need B >= 1, Tq >= 0, Hq >= 1, Hkv >= 1 (got %d, %d, %d, %d)",
                p->B, p->Tq, p->Hq, p->Hkv);
  if (p->Hq % p->Hkv) return fail(SKV_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->D != 64 && p->D != 128) return fail(SKV_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", p->D);
  if (!elem_bytes(p->dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", p->dtype);
  if (p->out_dtype != p->dtype && p->out_dtype != SKV_F32)
    return fail(SKV_ERR_DTYPE, "out_dtype must equal dtype or be SKV_F32");
  if (p->cap < 1) return fail(SKV_ERR_SHAPE, "cap must be >= 1 (got %d)", p->cap);
  if (p->mask < SKV_MASK_NONE || p->mask > SKV_MASK_BLOCK_CAUSAL)
    return fail(SKV_ERR_RANGE, "unknown mask %d", p->mask);
  if (p->mask == SKV_MASK_BLOCK_CAUSAL && p->mask_block < 1)
    return fail(SKV_ERR_RANGE, "mask_block must be >= 1 (got %d)", p->mask_block);
  if (p->flags & ~(unsigned)SKV_FULL_CAPACITY_MASKED) return fail(SKV_ERR_RANGE, "unknown flags 0x%x", p->flags);
  if (!(p->scale >= 0.f) || isinf(p->scale)) return fail(SKV_ERR_RANGE, "scale must be finite and >= 0");
  if (!packed && !p->kv_len_dev) {
    if (p->kv_len < 1 || p->kv_len > p->cap)
      return fail(SKV_ERR_RANGE, "kv_len=%d outside [1, cap=%d]", p->kv_len, p->cap);
    if (p->mask != SKV_MASK_NONE && p->Tq > p->kv_len)
      return fail(SKV_ERR_RANGE, "masked chunk of Tq=%d queries longer than kv_len=%d", p->Tq, p->kv_len);
  }
  if (p->max_seqlen_kv < 0) return fail(SKV_ERR_RANGE, "max_seqlen_kv must be >= 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(SKV_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  const int64_t elems = (int64_t)p->B * p->Tq * p->Hq;
  if (elems > 0x7fffffff) return fail(SKV_ERR_SHAPE, "B*Tq*Hq too large");
  // the kernels address a 64-row block of q, k, v or out rows with 32-bit byte offsets
  if ((int64_t)p->Hq * p->D > (1 << 21))
    return fail(SKV_ERR_SHAPE, "Hq*D=%lld too large (at most 2^21)", (long long)p->Hq * p->D);
  return SKV_OK;
}

// rotary-write arguments: frequency table, pair layout, a head size the kernels tile by
// (8 coordinate pairs per thread, 256 threads per workgroup)
skv_status check_rope(const double* inv_freq_dev, int rope_layout, int D) {
  if (!inv_freq_dev) return fail(SKV_ERR_NULL, "inv_freq_dev is NULL");
  if ((uintptr_t)inv_freq_dev & 7) return fail(SKV_ERR_ALIGN, "inv_freq_dev must be 8-byte aligned");
  if (rope_layout != SKV_ROPE_HALF && rope_layout != SKV_ROPE_INTERLEAVED)
    return fail(SKV_ERR_RANGE, "unknown rope_layout %d", rope_layout);
  if (D < 16 || D > 4096 || (D & (D - 1)))
    return fail(SKV_ERR_SHAPE, "rotary writes need D a power of two in [16, 4096] (got %d)", D);
  return SKV_OK;
}

}  // namespace

struct skv_ring {
  void* k_store;
  void* v_store;
  int32_t* meta;
  int B, chunk, n_slots, sink, Hkv, D, dtype;
  int vpr;  // 16-byte vectors per cache row
};

extern "C" {

const char* skv_last_error(void) { return g_err.c_str(); }
const char* skv_version(void) { return "libskv 0.1 (gfx950)"; }

skv_status kv_write_indexed(void* k_cache, void* v_cache, const void* k_src, const void* v_src,
                            const int64_t* index_dev, int64_t start, int B, int cap, int n,
                            int Hkv, int D, int dtype, int32_t* err_dev, void* stream) {
  if (!k_cache || !k_src) return fail(SKV_ERR_NULL, "k_cache and k_src must be non-NULL");
  if ((v_cache == nullptr) != (v_src == nullptr))
    return fail(SKV_ERR_NULL, "v_cache and v_src must both be given or both be NULL");
  if (!elem_bytes(dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B < 0 || n < 0 || cap < 1 || Hkv < 1 || D < 1)
    return fail(SKV_ERR_SHAPE, "bad sizes B=%d cap=%d n=%d Hkv=%d D=%d", B, cap, n, Hkv, D);
  const int64_t row_bytes = (int64_t)Hkv * D * elem_bytes(dtype);
  if (row_bytes % 16) return fail(SKV_ERR_ALIGN, "row of Hkv*D elements (%lld bytes) is not a multiple of 16", (long long)row_bytes);
  if (!aligned16(k_cache) || !aligned16(k_src) || !aligned16(v_cache) || !aligned16(v_src))
    return fail(SKV_ERR_ALIGN, "cache and source pointers must be 16-byte aligned");
  if (!index_dev && (start < 0 || start + n > cap))
    return fail(SKV_ERR_RANGE, "rows [%lld, %lld) outside the cache of %d rows", (long long)start,
                (long long)(start + n), cap);
  if ((int64_t)B * n > 0x7fffffff || (int64_t)n * (row_bytes / 16) > 0x7fffffff)
    return fail(SKV_ERR_SHAPE, "B*n or n*Hkv*D too large");
  if (B == 0 || n == 0) return ok();
  return hip_status(launch_write_indexed(k_src, v_src, k_cache, v_cache, index_dev, start, B, n,
                                         cap, (int)(row_bytes / 16), err_dev, (hipStream_t)stream),
                    "kv_write_indexed launch");
}

skv_status kv_write_indexed_rope(void* k_cache, void* v_cache, const void* k_src,
                                 const void* v_src, const int64_t* index_dev, int64_t start, int B,
                                 int cap, int n, int Hkv, int D, int dtype,
                                 const double* inv_freq_dev, int rope_layout, int32_t* err_dev,
                                 void* stream) {
  if (!k_cache || !k_src) return fail(SKV_ERR_NULL, "k_cache and k_src must be non-NULL");
  if ((v_cache == nullptr) != (v_src == nullptr))
    return fail(SKV_ERR_NULL, "v_cache and v_src must both be given or both be NULL");
  if (!elem_bytes(dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B < 0 || n < 0 || cap < 1 || Hkv < 1 || D < 1)
    return fail(SKV_ERR_SHAPE, "bad sizes B=%d cap=%d n=%d Hkv=%d D=%d", B, cap, n, Hkv, D);
  const skv_status rs = check_rope(inv_freq_dev, rope_layout, D);
  if (rs != SKV_OK) return rs;
  if (!aligned16(k_cache) || !aligned16(k_src) || !aligned16(v_cache) || !aligned16(v_src))
    return fail(SKV_ERR_ALIGN, "cache and source pointers must be 16-byte aligned");
  if (!index_dev && (start < 0 || start + n > cap))
    return fail(SKV_ERR_RANGE, "rows [%lld, %lld) outside the cache of %d rows", (long long)start,
                (long long)(start + n), cap);
  if ((int64_t)B * n > 0x7fffffff) return fail(SKV_ERR_SHAPE, "B*n too large");
  if (B == 0 || n == 0) return ok();
  return hip_status(launch_write_indexed_rope(k_src, v_src, k_cache, v_cache, index_dev, start, B,
                                              n, cap, Hkv, D, dtype, inv_freq_dev, rope_layout,
                                              err_dev, (hipStream_t)stream),
                    "kv_write_indexed_rope launch");
}

skv_status kv_cursor_advance(int32_t* cursor_dev, int n, int cap, int B, int64_t* index_out_dev,
                             int32_t* kv_len_out_dev, int32_t* err_dev, void* stream) {
  if (!cursor_dev || !index_out_dev) return fail(SKV_ERR_NULL, "cursor_dev and index_out_dev must be non-NULL");
  if (n < 1 || cap < 1 || B < 0) return fail(SKV_ERR_SHAPE, "need n >= 1, cap >= 1, B >= 0");
  if (((uintptr_t)cursor_dev & 3) || ((uintptr_t)index_out_dev & 7) || ((uintptr_t)kv_len_out_dev & 3))
    return fail(SKV_ERR_ALIGN, "misaligned cursor / index / kv_len pointer");
  return hip_status(launch_cursor_advance(cursor_dev, n, cap, B, index_out_dev, kv_len_out_dev,
                                          err_dev, (hipStream_t)stream),
                    "kv_cursor_advance launch");
}

size_t kv_ring_meta_bytes(int B) { return B > 0 ? (size_t)B * 4 * sizeof(int32_t) : 0; }

skv_status kv_ring_create(skv_ring** out, void* k_store, void* v_store, void* meta_dev, int B,
                          int chunk, int n_slots, int sink_slots, int Hkv, int D, int dtype,
                          void* stream) {
  if (!out || !k_store || !meta_dev) return fail(SKV_ERR_NULL, "out, k_store and meta_dev must be non-NULL");
  *out = nullptr;
  if (!elem_bytes(dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B < 1 || chunk < 1 || Hkv < 1 || D < 1) return fail(SKV_ERR_SHAPE, "bad ring sizes");
  if (n_slots < 1 || sink_slots < 0 || sink_slots >= n_slots)
    return fail(SKV_ERR_RANGE, "need 0 <= sink_slots (%d) < n_slots (%d)", sink_slots, n_slots);
  if ((int64_t)n_slots * chunk > 0x7fffffff || (int64_t)B * chunk > 0x7fffffff)
    return fail(SKV_ERR_SHAPE, "ring too large");
  const int64_t row_bytes = (int64_t)Hkv * D * elem_bytes(dtype);
  if (row_bytes % 16) return fail(SKV_ERR_ALIGN, "row bytes not a multiple of 16");
  if ((int64_t)chunk * (row_bytes / 16) > 0x7fffffff) return fail(SKV_ERR_SHAPE, "chunk too large");
  if (!aligned16(k_store) || !aligned16(v_store) || ((uintptr_t)meta_dev & 3))
    return fail(SKV_ERR_ALIGN, "misaligned ring storage or metadata");
  skv_ring* r = (skv_ring*)malloc(sizeof(skv_ring));
  if (!r) return fail(SKV_ERR_RANGE, "out of host memory");
  *r = skv_ring{k_store, v_store, (int32_t*)meta_dev, B, chunk, n_slots, sink_slots, Hkv, D, dtype,
                (int)(row_bytes / 16)};
  hipError_t e = launch_ring_reset(r->meta, B, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) {
    free(r);
    return hip_status(e, "kv_ring_create launch");
  }
  *out = r;
  return ok();
}

skv_status kv_ring_reserve(skv_ring* r, const uint8_t* batch_mask_dev, void* stream) {
  if (!r) return fail(SKV_ERR_NULL, "ring is NULL");
  return hip_status(launch_ring_reserve(r->meta, r->B, batch_mask_dev, r->n_slots, r->sink,
                                        (hipStream_t)stream),
                    "kv_ring_reserve launch");
}

skv_status kv_ring_write(skv_ring* r, const void* k_src, const void* v_src,
                         const uint8_t* batch_mask_dev, int32_t* err_dev, void* stream) {
  if (!r) return fail(SKV_ERR_NULL, "ring is NULL");
  if (!k_src) return fail(SKV_ERR_NULL, "k_src is NULL");
  if ((r->v_store == nullptr) != (v_src == nullptr))
    return fail(SKV_ERR_NULL, "v_src must be given iff the ring has V storage");
  if (!aligned16(k_src) || !aligned16(v_src)) return fail(SKV_ERR_ALIGN, "sources must be 16-byte aligned");
  return hip_status(launch_ring_write(k_src, v_src, r->k_store, r->v_store, r->meta, r->B,
                                      batch_mask_dev, r->chunk, r->n_slots, r->vpr, err_dev,
                                      (hipStream_t)stream),
                    "kv_ring_write launch");
}

skv_status kv_ring_write_rope(skv_ring* r, const void* k_src, const void* v_src,
                              const double* inv_freq_dev, int rope_layout,
                              const uint8_t* batch_mask_dev, int32_t* err_dev, void* stream) {
  if (!r) return fail(SKV_ERR_NULL, "ring is NULL");
  if (!k_src) return fail(SKV_ERR_NULL, "k_src is NULL");
  if ((r->v_store == nullptr) != (v_src == nullptr))
    return fail(SKV_ERR_NULL, "v_src must be given iff the ring has V storage");
  const skv_status rs = check_rope(inv_freq_dev, rope_layout, r->D);
  if (rs != SKV_OK) return rs;
  if (!aligned16(k_src) || !aligned16(v_src)) return fail(SKV_ERR_ALIGN, "sources must be 16-byte aligned");
  return hip_status(launch_ring_write_rope(k_src, v_src, r->k_store, r->v_store, r->meta, r->B,
                                           batch_mask_dev, r->chunk, r->n_slots, r->Hkv, r->D,
                                           r->dtype, inv_freq_dev, rope_layout, err_dev,
                                           (hipStream_t)stream),
                    "kv_ring_write_rope launch");
}

skv_status kv_ring_reset(skv_ring* r, const uint8_t* batch_mask_dev, void* stream) {
  if (!r) return fail(SKV_ERR_NULL, "ring is NULL");
  return hip_status(launch_ring_reset(r->meta, r->B, batch_mask_dev, (hipStream_t)stream),
                    "kv_ring_reset launch");
}

const int32_t* kv_ring_kv_len_dev(const skv_ring* r) { return r ? r->meta + 3 * r->B : nullptr; }
const int32_t* kv_ring_slot_dev(const skv_ring* r) { return r ? r->meta + r->B : nullptr; }

skv_status kv_ring_destroy(skv_ring* r) {
  free(r);
  return ok();
}

skv_status kv_roll_left(void* k_store, void* v_store, int B, int rows, int sink_rows,
                        int shift_rows, int Hkv, int D, int dtype, void* stream) {
  if (!k_store) return fail(SKV_ERR_NULL, "k_store must be non-NULL");
  if (!elem_bytes(dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B < 0 || rows < 1 || Hkv < 1 || D < 1) return fail(SKV_ERR_SHAPE, "bad sizes");
  if (sink_rows < 0 || shift_rows < 1 || (int64_t)sink_rows + shift_rows > rows)
    return fail(SKV_ERR_RANGE, "need 0 <= sink_rows, 1 <= shift_rows, sink_rows + shift_rows <= rows "
                "(got %d, %d, %d)", sink_rows, shift_rows, rows);
  const int64_t row_bytes = (int64_t)Hkv * D * elem_bytes(dtype);
  if (row_bytes % 16) return fail(SKV_ERR_ALIGN, "row bytes not a multiple of 16");
  if (!aligned16(k_store) || !aligned16(v_store)) return fail(SKV_ERR_ALIGN, "misaligned storage");
  if ((int64_t)shift_rows * (row_bytes / 16) > 0x7fffffff) return fail(SKV_ERR_SHAPE, "shift too large");
  if (B == 0 || sink_rows + shift_rows == rows) return ok();
  return hip_status(launch_roll_left(k_store, v_store, B, rows, sink_rows, shift_rows,
                                     (int)(row_bytes / 16), (hipStream_t)stream),
                    "kv_roll_left launch");
}

skv_status kv_ragged_metadata(const int32_t* lens_dev, int B, int max_kv, int32_t* cu_seqlens_out_dev,
                              int32_t* err_dev, void* stream) {
  if (!lens_dev || !cu_seqlens_out_dev) return fail(SKV_ERR_NULL, "lens_dev and cu_seqlens_out_dev must be non-NULL");
  if (B < 1 || max_kv < 0) return fail(SKV_ERR_SHAPE, "need B >= 1, max_kv >= 0");
  if ((int64_t)B * max_kv > 0x7fffffff) return fail(SKV_ERR_SHAPE, "B*max_kv too large");
  if (((uintptr_t)lens_dev & 3) || ((uintptr_t)cu_seqlens_out_dev & 3))
    return fail(SKV_ERR_ALIGN, "misaligned lens / cu_seqlens");
  return hip_status(launch_ragged_metadata(lens_dev, B, max_kv, cu_seqlens_out_dev, err_dev,
                                           (hipStream_t)stream),
                    "kv_ragged_metadata launch");
}

skv_status kv_pack_ragged(void* k_packed, void* v_packed, const void* k_padded, const void* v_padded,
                          const int32_t* cu_seqlens_dev, int B, int max_kv, int packed_rows, int Hkv,
                          int D, int dtype, int32_t* err_dev, void* stream) {
  const bool no_rows = packed_rows == 0;  // packed buffers may then be NULL (nothing is written)
  if (!k_padded || !cu_seqlens_dev || (!k_packed && !no_rows))
    return fail(SKV_ERR_NULL, "k_packed, k_padded and cu_seqlens_dev must be non-NULL");
  if (!no_rows && (v_packed == nullptr) != (v_padded == nullptr))
    return fail(SKV_ERR_NULL, "v_packed and v_padded must both be given or both be NULL");
  if (!elem_bytes(dtype)) return fail(SKV_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B < 1 || max_kv < 0 || packed_rows < 0 || Hkv < 1 || D < 1)
    return fail(SKV_ERR_SHAPE, "bad sizes B=%d max_kv=%d packed_rows=%d Hkv=%d D=%d", B, max_kv,
                packed_rows, Hkv, D);
  const int64_t row_bytes = (int64_t)Hkv * D * elem_bytes(dtype);
  if (row_bytes % 16) return fail(SKV_ERR_ALIGN, "row bytes not a multiple of 16");
  if (!aligned16(k_packed) || !aligned16(v_packed) || !aligned16(k_padded) || !aligned16(v_padded) ||
      ((uintptr_t)cu_seqlens_dev & 3))
    return fail(SKV_ERR_ALIGN, "misaligned buffers");
  if ((int64_t)max_kv * (row_bytes / 16) > 0x7fffffff) return fail(SKV_ERR_SHAPE, "max_kv too large");
  if (max_kv == 0) return ok();
  return hip_status(launch_pack_ragged(k_padded, v_padded, k_packed, v_packed, cu_seqlens_dev, B,
                                       max_kv, packed_rows, (int)(row_bytes / 16), err_dev,
                                       (hipStream_t)stream),
                    "kv_pack_ragged launch");
}

size_t attn_workspace_bytes(const skv_attn_params* p) {
  if (!p) {
    fail(SKV_ERR_NULL, "params is NULL");
    return (size_t)-1;
  }
  if (validate_attn((void*)16, (void*)16, (void*)16, (void*)16, p) != SKV_OK) return (size_t)-1;
  ok();
  if (choose_path(*p) == PATH_F32) return 0;
  if (choose_path(*p) == PATH_FLASH) return flash_workspace_bytes(p->B, p->Hq, p->Tq, p->D, key_bound(*p));
  const int splits = decode_splits(p->B, p->Hkv, key_bound(*p));
  return decode_workspace_bytes(p->B, p->Hkv, p->D, splits);
}

skv_status attn_chunk_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          const skv_attn_params* p, void* stream) {
  skv_status st = validate_attn(q, k, v, out, p);
  if (st != SKV_OK) return st;
  if (lse && ((uintptr_t)lse & 3)) return fail(SKV_ERR_ALIGN, "lse must be 4-byte aligned");
  if (p->Tq == 0) return ok();
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.kv_len_dev = p->kv_len_dev;
  a.cu = p->cu_seqlens_kv_dev;
  a.err = p->err_dev;
  a.B = p->B;
  a.Tq = p->Tq;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.cap = p->cap;
  a.kv_len_host = p->kv_len;
  a.mask = p->mask;
  a.block = p->mask == SKV_MASK_BLOCK_CAUSAL ? p->mask_block : 1;
  a.full_cap = (p->flags & SKV_FULL_CAPACITY_MASKED) ? 1 : 0;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  switch (choose_path(*p)) {
    case PATH_F32:
      return hip_status(launch_attn_f32(a, p->D, s), "attn_chunk_fwd (fp32) launch");
    case PATH_FLASH:
      return hip_status(launch_attn_flash(a, p->dtype, p->out_dtype, p->D, key_bound(*p),
                                          p->workspace, p->workspace_bytes, s),
                        "attn_chunk_fwd (flash) launch");
    case PATH_DECODE: {
      const int splits = decode_splits(p->B, p->Hkv, key_bound(*p));
      const size_t need = decode_workspace_bytes(p->B, p->Hkv, p->D, splits);
      if (!p->workspace) return fail(SKV_ERR_NULL, "decode-sized call needs a workspace of %zu bytes", need);
      if (p->workspace_bytes < need)
        return fail(SKV_ERR_RANGE, "workspace of %zu bytes < %zu required", p->workspace_bytes, need);
      if (!aligned16(p->workspace)) return fail(SKV_ERR_ALIGN, "workspace must be 16-byte aligned");
      return hip_status(launch_attn_decode(a, p->dtype, p->out_dtype, p->D, p->workspace, splits,
                                           key_bound(*p), s),
                        "attn_chunk_fwd (decode) launch");
    }
  }
  return fail(SKV_ERR_UNSUPPORTED, "no path");
}

}  // extern "C"

namespace {

// Checks shared by both fused decode entry points; on success *splits and *bound hold the launch
// plan and *need the workspace bytes it takes.
skv_status check_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                             int32_t* kv_len_out_dev, const skv_attn_params* p, int* splits,
                             int* bound, size_t* need) {
  if (!p) return fail(SKV_ERR_NULL, "params is NULL");
  if (!k_new || !v_new || !cursor_dev) return fail(SKV_ERR_NULL, "k_new, v_new and cursor_dev must be non-NULL");
  if (p->kv_len_dev || p->cu_seqlens_kv_dev || (p->flags & SKV_FULL_CAPACITY_MASKED))
    return fail(SKV_ERR_UNSUPPORTED, "the fused decode step takes its length from the cursor "
                                     "(no kv_len_dev, cu_seqlens_kv_dev or full-capacity arm)");
  skv_attn_params v = *p;
  v.kv_len = v.cap;  // any valid host length: the kernel reads the cursor instead
  if (v.mask != SKV_MASK_NONE && v.Tq > v.kv_len) v.kv_len = v.Tq;
  skv_status st = validate_attn(q, k_cache, v_cache, out, &v);
  if (st != SKV_OK) return st;
  if (p->Tq > 0 && choose_path(v) != PATH_DECODE)
    return fail(SKV_ERR_UNSUPPORTED, "the fused decode step needs bf16/f16, Tq <= %d, "
                "Tq*Hq/Hkv <= %d and B*Hkv < %d", kDecodeMaxTq, kDecodeMaxRows, kWsCounterInts);
  if (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)cursor_dev & 3) ||
      ((uintptr_t)kv_len_out_dev & 3) || (lse && ((uintptr_t)lse & 3)))
    return fail(SKV_ERR_ALIGN, "misaligned k_new / v_new / cursor / kv_len_out / lse");
  *bound = p->max_seqlen_kv > 0 && p->max_seqlen_kv < p->cap ? p->max_seqlen_kv : p->cap;
  *splits = decode_splits(p->B, p->Hkv, *bound);
  *need = decode_workspace_bytes(p->B, p->Hkv, p->D, *splits);
  return SKV_OK;
}

skv_status launch_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                              int32_t* kv_len_out_dev, const skv_attn_params* p, void* ws,
                              int splits, int bound, hipStream_t stream, const char* what) {
  AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.lse = lse;
  a.err = p->err_dev;
  a.B = p->B;
  a.Tq = p->Tq;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.cap = p->cap;
  a.mask = p->mask;
  a.block = p->mask == SKV_MASK_BLOCK_CAUSAL ? p->mask_block : 1;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cursor = cursor_dev;
  a.kv_len_out = kv_len_out_dev;
  return hip_status(launch_attn_decode(a, p->dtype, p->out_dtype, p->D, ws, splits, bound, stream), what);
}

}  // namespace

extern "C" {

skv_status attn_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                            void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                            int32_t* kv_len_out_dev, const skv_attn_params* p, void* stream) {
  int splits = 0, bound = 0;
  size_t need = 0;
  skv_status st = check_decode_step(q, k_new, v_new, k_cache, v_cache, out, lse, cursor_dev,
                                    kv_len_out_dev, p, &splits, &bound, &need);
  if (st != SKV_OK) return st;
  if (p->Tq == 0) return ok();
  if (!p->workspace) return fail(SKV_ERR_NULL, "the decode step needs a workspace of %zu bytes", need);
  if (p->workspace_bytes < need)
    return fail(SKV_ERR_RANGE, "workspace of %zu bytes < %zu required", p->workspace_bytes, need);
  if (!aligned16(p->workspace)) return fail(SKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  return launch_decode_step(q, k_new, v_new, k_cache, v_cache, out, lse, cursor_dev, kv_len_out_dev, p,
                            p->workspace, splits, bound, (hipStream_t)stream, "attn_decode_step launch");
}

// ---------------------------------------------------------------------------------------
// Fused decode step without a caller workspace
// ---------------------------------------------------------------------------------------
}  // extern "C"

// The split-K scratch of attn_decode_step_static: arrival counters (the first kWsCounterInts
// ints, zero between calls) and partials. Each GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` is only a stand-in for the symbol: the device
// address of this GPU's copy comes from hipGetSymbolAddress and is the only form used.
static __device__ __align__(256) unsigned char scratch[SKV_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = SKV_DECODE_STATIC_SCRATCH_BYTES;

__global__ void k_zero_ints(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once set up

// This device's scratch address; the first call on a device looks it up (with that device
// current) and clears the counter area by a kernel on `stream` (not a memset, which a graph
// capture would record as a memset node).
skv_status device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SKV_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    hipLaunchKernelGGL(k_zero_ints, dim3(64), dim3(256), 0, stream, (int*)ptr, kWsCounterInts);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "clearing the static scratch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

}  // namespace

extern "C" {

skv_status attn_decode_step_static(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                                   int32_t* kv_len_out_dev, const skv_attn_params* p, void* stream) {
  int splits = 0, bound = 0;
  size_t need = 0;
  skv_status st = check_decode_step(q, k_new, v_new, k_cache, v_cache, out, lse, cursor_dev,
                                    kv_len_out_dev, p, &splits, &bound, &need);
  if (st != SKV_OK) return st;
  if (need > kStaticScratchBytes)
    return fail(SKV_ERR_RANGE, "this decode step needs %zu bytes of split-K scratch; the static scratch "
                "holds %zu (B*Hkv and the key bound set the need)", need, kStaticScratchBytes);
  if (p->Tq == 0) return ok();
  void* ws = nullptr;
  st = device_scratch((hipStream_t)stream, &ws);
  if (st != SKV_OK) return st;
  return launch_decode_step(q, k_new, v_new, k_cache, v_cache, out, lse, cursor_dev, kv_len_out_dev, p,
                            ws, splits, bound, (hipStream_t)stream, "attn_decode_step_static launch");
}

// ---------------------------------------------------------------------------------------
// Measurement probes
// ---------------------------------------------------------------------------------------
skv_status skv_probe_mfma_bf16(float* out_dev, int workgroups, int iters, void* stream) {
  if (!out_dev) return fail(SKV_ERR_NULL, "out_dev is NULL");
  if (workgroups < 1 || iters < 1) return fail(SKV_ERR_RANGE, "need workgroups >= 1 and iters >= 1");
  if ((uintptr_t)out_dev & 3) return fail(SKV_ERR_ALIGN, "out_dev must be 4-byte aligned");
  return hip_status(launch_peak_mfma_bf16(out_dev, workgroups, iters, (hipStream_t)stream),
                    "skv_probe_mfma_bf16 launch");
}

skv_status skv_probe_copy(void* dst_dev, const void* src_dev, size_t bytes, void* stream) {
  if (!dst_dev || !src_dev) return fail(SKV_ERR_NULL, "dst_dev and src_dev must be non-NULL");
  if (bytes % 16) return fail(SKV_ERR_SHAPE, "bytes must be a multiple of 16 (got %zu)", bytes);
  if (!aligned16(dst_dev) || !aligned16(src_dev)) return fail(SKV_ERR_ALIGN, "buffers must be 16-byte aligned");
  if (bytes / 16 / 512 >= 0x7fffffffu) return fail(SKV_ERR_SHAPE, "copy too large");
  if (bytes == 0) return ok();
  return hip_status(launch_peak_copy(dst_dev, src_dev, bytes, (hipStream_t)stream), "skv_probe_copy launch");
}

}  // extern "C"
