// KV-cache write kernels: indexed slab rows, the device write cursor, and the
// sink-plus-window ring (reserve / write / reset).
//
// Sources: LingBot-World PR #53 "refactor(kv): index_copy_ for KV-cache writes (enabler for
// multi-user batching + CUDA Graphs)" (Summary: index_copy along the sequence dim with one
// index vector for the whole batch) and flashdreams issue #763 "add an opt-in circular KV
// policy for streaming attention" (proposed boundary: fixed slots, reservation separate from
// writes, pinned sink, device-resident slot metadata).
//
// A cache row (one token, all KV heads) is Hkv*D elements, contiguous: 0.5-10 KiB. The
// source block of one batch element, [n, Hkv, D], is contiguous too, so each workgroup moves
// an 8 KiB span of it (256 threads x 2 vectors of 16 bytes, both loads issued before the first
// store) whatever the row size; each vector finds its destination row from its position
// (longer spans per workgroup measured slower: 32 KiB spans halved the slab write rate). For
// the ring the destination of a batch element's chunk is also one contiguous span (its slot),
// so that write is a plain span copy with the slot read once per workgroup. The kernels are
// HBM-bound: each byte is read once and written once.
#include "common.h"
#include "ring_meta.h"

namespace skv {

constexpr int kCopyThreads = 256;
constexpr int kCopyPer = 2;                           // 16-byte vectors per thread
constexpr int kCopySpan = kCopyThreads * kCopyPer;    // vectors per workgroup (8 KiB)

// index_copy along dim 1: cache[b, index[t]] = src[b, t] (index == nullptr: start + t).
// Grid: (B * spans per batch element, tensors). Vector i of batch element b's source block is
// row t = i / vpr, column i % vpr; it goes to row index[t] of b's cache.
__global__ void __launch_bounds__(kCopyThreads)
k_write_indexed(const i32x4* __restrict__ k_src, const i32x4* __restrict__ v_src,
                i32x4* __restrict__ k_cache, i32x4* __restrict__ v_cache,
                const int64_t* __restrict__ index, int64_t start, int n, int cap, int vpr,
                int spans, int32_t* err) {
  const int b = blockIdx.x / spans;
  const int span = blockIdx.x - b * spans;
  const bool is_v = blockIdx.y != 0;
  const int nv = n * vpr;  // vectors per batch element (host-checked to fit an int)
  const i32x4* src = (is_v ? v_src : k_src) + (int64_t)b * nv;
  i32x4* cache = (is_v ? v_cache : k_cache) + (int64_t)b * cap * vpr;
  const int i0 = span * kCopySpan + threadIdx.x;
  i32x4 r[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) r[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i >= nv) continue;
    const int t = i / vpr;
    const int col = i - t * vpr;
    const int64_t dst_row = index ? index[t] : start + t;
    if (dst_row < 0 || dst_row >= cap) {
      if (!is_v && col == 0) report(err, SKV_DEV_INDEX_RANGE);
      continue;
    }
    cache[dst_row * vpr + col] = r[u];
  }
}

// Device cursor: index[t] = c + t, kv_len[b] = c + n, cursor = c + n (if it fits).
__global__ void __launch_bounds__(256)
k_cursor_advance(int32_t* cursor, int n, int cap, int B, int64_t* index_out, int32_t* kv_len_out,
                 int32_t* err) {
  const int c = *cursor;
  const bool fits = c >= 0 && (int64_t)c + n <= cap;
  for (int t = threadIdx.x; t < n; t += blockDim.x) index_out[t] = fits ? (int64_t)c + t : -1;
  if (fits && kv_len_out)
    for (int b = threadIdx.x; b < B; b += blockDim.x) kv_len_out[b] = c + n;
  __syncthreads();  // every thread has read the cursor before it moves
  if (threadIdx.x == 0) {
    if (fits) *cursor = c + n;
    else report(err, SKV_DEV_CURSOR_FULL);
  }
}

// ---------------------------------------------------------------------------------------
// Ring (metadata layout and helpers in ring_meta.h)
// ---------------------------------------------------------------------------------------

// Reset (also the initialisation): forget every chunk, keep the storage untouched.
__global__ void k_ring_reset(int32_t* meta, int B, const uint8_t* mask) {
  RingMeta m = ring_meta(meta, B);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    if (!selected(mask, b)) continue;
    m.counter[b] = 0;
    m.slot[b] = -1;
    m.pending[b] = 0;
    m.valid[b] = 0;
  }
}

// Reserve the slot of the next chunk. The first `sink` chunks since reset are pinned; once
// all n_slots are full, chunk c replaces the oldest non-sink chunk, which sits in slot
// sink + (c - sink) mod (n_slots - sink). A reservation not yet written is kept.
__global__ void k_ring_reserve(int32_t* meta, int B, const uint8_t* mask, int n_slots, int sink) {
  RingMeta m = ring_meta(meta, B);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    if (!selected(mask, b) || m.pending[b]) continue;
    const int c = m.counter[b];
    m.slot[b] = c < n_slots ? c : sink + (c - sink) % (n_slots - sink);
    m.counter[b] = c + 1;
    m.pending[b] = 1;
  }
}

// Write the current chunk [B, C, Hkv, D] into its reserved slot. Block (0,0) also commits the
// retained-token count at the first write after a reserve; every other block only reads
// slot[], which no block of this launch modifies. Grid: (B * spans per chunk, tensors); a
// batch element's chunk and its slot's rows are both contiguous, so this is a span copy.
__global__ void __launch_bounds__(kCopyThreads)
k_ring_write(const i32x4* __restrict__ k_src, const i32x4* __restrict__ v_src,
             i32x4* __restrict__ k_store, i32x4* __restrict__ v_store, int32_t* meta, int B,
             const uint8_t* mask, int C, int n_slots, int vpr, int spans, int32_t* err) {
  RingMeta m = ring_meta(meta, B);
  if (blockIdx.x == 0 && blockIdx.y == 0) ring_commit(m, B, mask, C, n_slots, err);
  const int b = blockIdx.x / spans;
  const int span = blockIdx.x - b * spans;
  if (!selected(mask, b)) return;
  const int s = m.slot[b];
  if (s < 0 || s >= n_slots) return;  // unreserved (reported by block 0) or corrupt metadata
  const bool is_v = blockIdx.y != 0;
  const int nv = C * vpr;  // vectors per chunk (checked to fit an int when the ring was made)
  const i32x4* src = (is_v ? v_src : k_src) + (int64_t)b * nv;
  i32x4* dst = (is_v ? v_store : k_store) + ((int64_t)b * n_slots + s) * nv;
  const int i0 = span * kCopySpan + threadIdx.x;
  i32x4 r[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) r[u] = __builtin_nontemporal_load(src + i);
  }
  // nontemporal stores: back-to-back chunk writes ran 7% faster with them (no change with a
  // flushed cache before each write); the slab write measured slower cold with them
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) __builtin_nontemporal_store(r[u], dst + i);
  }
}

// ---------------------------------------------------------------------------------------
// Chronological window roll-left (comparison arm) and ragged K/V packing
// ---------------------------------------------------------------------------------------

// Block move per batch element: vectors [0, nv) of src + b * src_stride go to dst + b *
// dst_stride; the caller guarantees that source and destination do not overlap.
__global__ void __launch_bounds__(kCopyThreads)
k_move_block(const i32x4* __restrict__ k_src, i32x4* __restrict__ k_dst, const i32x4* v_src,
             i32x4* v_dst, int64_t src_stride, int64_t dst_stride, int nv, int spans) {
  const int b = blockIdx.x / spans;
  const int span = blockIdx.x - b * spans;
  const bool is_v = blockIdx.y != 0;
  const i32x4* src = (is_v ? v_src : k_src) + (int64_t)b * src_stride;
  i32x4* dst = (is_v ? v_dst : k_dst) + (int64_t)b * dst_stride;
  const int i0 = span * kCopySpan + threadIdx.x;
  i32x4 r[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) r[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) dst[i] = r[u];
  }
}

// cu[0] = 0, cu[b+1] = cu[b] + len_b, lengths outside [0, max_kv] counted as 0 (flagged).
__global__ void k_ragged_metadata(const int32_t* lens, int B, int max_kv, int32_t* cu, int32_t* err) {
  if (threadIdx.x != 0) return;
  int64_t acc = 0;
  cu[0] = 0;
  bool bad = false;
  for (int b = 0; b < B; ++b) {
    int l = lens[b];
    if (l < 0 || l > max_kv) {
      bad = true;
      l = 0;
    }
    acc += l;
    cu[b + 1] = (int32_t)acc;
  }
  if (bad) report(err, SKV_DEV_KV_LEN);
}

// Packing: vector i of batch element b's padded block is row t = i / vpr; rows t < len_b go
// to packed row cu[b] + t. Grid: (B * spans over max_kv rows, tensors).
__global__ void __launch_bounds__(kCopyThreads)
k_pack_ragged(const i32x4* __restrict__ k_pad, const i32x4* __restrict__ v_pad,
              i32x4* __restrict__ k_pack, i32x4* __restrict__ v_pack, const int32_t* cu, int max_kv,
              int packed_rows, int vpr, int spans, int32_t* err) {
  const int b = blockIdx.x / spans;
  const int span = blockIdx.x - b * spans;
  const bool is_v = blockIdx.y != 0;
  const int lo = cu[b], len = cu[b + 1] - lo;
  if (lo < 0 || len < 0 || len > max_kv || (int64_t)lo + len > packed_rows) {
    if (!is_v && span == 0 && threadIdx.x == 0) report(err, SKV_DEV_CU_SEQLENS);
    return;
  }
  const int nv = len * vpr;  // only the valid rows are read
  const i32x4* src = (is_v ? v_pad : k_pad) + (int64_t)b * max_kv * vpr;
  i32x4* dst = (is_v ? v_pack : k_pack) + (int64_t)lo * vpr;
  const int i0 = span * kCopySpan + threadIdx.x;
  i32x4 r[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) r[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int i = i0 + u * kCopyThreads;
    if (i < nv) dst[i] = r[u];
  }
}

// ---------------------------------------------------------------------------------------
// Host launchers (called by api.hip after argument validation)
// ---------------------------------------------------------------------------------------
static int copy_spans(int64_t vectors) { return (int)((vectors + kCopySpan - 1) / kCopySpan); }

hipError_t launch_write_indexed(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                                const int64_t* index, int64_t start, int B, int n, int cap,
                                int vpr, int32_t* err, hipStream_t s) {
  const int spans = copy_spans((int64_t)n * vpr);
  dim3 grd((unsigned)((int64_t)B * spans), v_cache ? 2 : 1);
  hipLaunchKernelGGL(k_write_indexed, grd, dim3(kCopyThreads), 0, s, (const i32x4*)k_src,
                     (const i32x4*)v_src, (i32x4*)k_cache, (i32x4*)v_cache, index, start, n, cap,
                     vpr, spans, err);
  return hipGetLastError();
}

hipError_t launch_cursor_advance(int32_t* cursor, int n, int cap, int B, int64_t* index_out,
                                 int32_t* kv_len_out, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(k_cursor_advance, dim3(1), dim3(256), 0, s, cursor, n, cap, B, index_out,
                     kv_len_out, err);
  return hipGetLastError();
}

hipError_t launch_ring_reset(int32_t* meta, int B, const uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(k_ring_reset, dim3(1), dim3(256), 0, s, meta, B, mask);
  return hipGetLastError();
}

hipError_t launch_ring_reserve(int32_t* meta, int B, const uint8_t* mask, int n_slots, int sink,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_ring_reserve, dim3(1), dim3(256), 0, s, meta, B, mask, n_slots, sink);
  return hipGetLastError();
}

hipError_t launch_ring_write(const void* k_src, const void* v_src, void* k_store, void* v_store,
                             int32_t* meta, int B, const uint8_t* mask, int C, int n_slots,
                             int vpr, int32_t* err, hipStream_t s) {
  const int spans = copy_spans((int64_t)C * vpr);
  dim3 grd((unsigned)((int64_t)B * spans), v_store ? 2 : 1);
  hipLaunchKernelGGL(k_ring_write, grd, dim3(kCopyThreads), 0, s, (const i32x4*)k_src,
                     (const i32x4*)v_src, (i32x4*)k_store, (i32x4*)v_store, meta, B, mask, C,
                     n_slots, vpr, spans, err);
  return hipGetLastError();
}

hipError_t launch_roll_left(void* k_store, void* v_store, int B, int rows, int sink_rows,
                            int shift_rows, int vpr, hipStream_t s) {
  // Pieces of at most shift_rows rows, in increasing row order: piece p reads rows that no
  // earlier piece writes and writes rows that earlier pieces have already read (stream order),
  // so the overlapping move needs no staging copy.
  const int64_t stride = (int64_t)rows * vpr;
  for (int first = sink_rows + shift_rows; first < rows; first += shift_rows) {
    const int n = rows - first < shift_rows ? rows - first : shift_rows;
    const int nv = n * vpr;
    const int spans = copy_spans(nv);
    dim3 grd((unsigned)((int64_t)B * spans), v_store ? 2 : 1);
    const i32x4* ks = (const i32x4*)k_store + (int64_t)first * vpr;
    i32x4* kd = (i32x4*)k_store + (int64_t)(first - shift_rows) * vpr;
    const i32x4* vs = v_store ? (const i32x4*)v_store + (int64_t)first * vpr : nullptr;
    i32x4* vd = v_store ? (i32x4*)v_store + (int64_t)(first - shift_rows) * vpr : nullptr;
    hipLaunchKernelGGL(k_move_block, grd, dim3(kCopyThreads), 0, s, ks, kd, vs, vd, stride, stride,
                       nv, spans);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ragged_metadata(const int32_t* lens, int B, int max_kv, int32_t* cu, int32_t* err,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_ragged_metadata, dim3(1), dim3(64), 0, s, lens, B, max_kv, cu, err);
  return hipGetLastError();
}

hipError_t launch_pack_ragged(const void* k_pad, const void* v_pad, void* k_pack, void* v_pack,
                              const int32_t* cu, int B, int max_kv, int packed_rows, int vpr,
                              int32_t* err, hipStream_t s) {
  const int spans = copy_spans((int64_t)max_kv * vpr);
  dim3 grd((unsigned)((int64_t)B * spans), v_pack ? 2 : 1);
  hipLaunchKernelGGL(k_pack_ragged, grd, dim3(kCopyThreads), 0, s, (const i32x4*)k_pad,
                     (const i32x4*)v_pad, (i32x4*)k_pack, (i32x4*)v_pack, cu, max_kv, packed_rows,
                     vpr, spans, err);
  return hipGetLastError();
}

}  // namespace skv
