// KV-cache write kernels: indexed slab rows, the device write cursor, and the
// sink-plus-window ring (reserve / write / reset).
//
// Sources: LingBot-World PR #53 "refactor(kv): index_copy_ for KV-cache writes (enabler for
// multi-user batching + CUDA Graphs)" (Summary: index_copy along the sequence dim with one
// index vector for the whole batch) and flashdreams issue #763 "add an opt-in circular KV
// policy for streaming attention" (proposed boundary: fixed slots, reservation separate from
// writes, pinned sink, device-resident slot metadata).
//
// A cache row (one token, all KV heads) is Hkv*D elements, contiguous: 0.5-10 KiB. Each
// workgroup moves one source row of one tensor with 16-byte loads/stores; the grid is
// (rows, tensors, chunks of 1024 vectors), so no per-element division is needed and every
// wavefront issues fully coalesced 1 KiB accesses. The kernels are HBM-bound: each byte is
// read once and written once.
#include "common.h"

namespace skv {

constexpr int kCopyUnroll = 4;

// Copy source row `row` (of n rows per batch element) to destination row `dst_row` of batch
// element b. Vectors [blockIdx.z*blockDim*U, ...) of the row are handled by this block.
__device__ __forceinline__ void copy_row(const uint4* __restrict__ src_, uint4* __restrict__ dst_,
                                         int vpr) {
  const i32x4* src = (const i32x4*)src_;  // native vector type for the nontemporal builtin
  i32x4* dst = (i32x4*)dst_;
  const int v0 = blockIdx.z * blockDim.x * kCopyUnroll + threadIdx.x;
  i32x4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    int v = v0 + u * blockDim.x;
    if (v < vpr) r[u] = __builtin_nontemporal_load(src + v);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    int v = v0 + u * blockDim.x;
    if (v < vpr) dst[v] = r[u];
  }
}

// index_copy along dim 1: cache[b, index[t]] = src[b, t] (index == nullptr: start + t).
__global__ void __launch_bounds__(256)
k_write_indexed(const uint4* __restrict__ k_src, const uint4* __restrict__ v_src,
                uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                const int64_t* __restrict__ index, int64_t start, int n, int cap, int vpr,
                int32_t* err) {
  const int row = blockIdx.x;  // b * n + t
  const int b = row / n;
  const int t = row - b * n;
  const bool is_v = blockIdx.y != 0;
  const int64_t dst_row = index ? index[t] : start + t;
  if (dst_row < 0 || dst_row >= cap) {
    if (!is_v && blockIdx.z == 0 && threadIdx.x == 0) report(err, SKV_DEV_INDEX_RANGE);
    return;
  }
  const uint4* src = (is_v ? v_src : k_src) + (int64_t)row * vpr;
  uint4* dst = (is_v ? v_cache : k_cache) + ((int64_t)b * cap + dst_row) * vpr;
  copy_row(src, dst, vpr);
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
// Ring metadata: int32 [4][B] = counter, slot, pending, valid (structure of arrays, so
// valid[] is directly the [B] kv_len vector attention reads).
// ---------------------------------------------------------------------------------------
struct RingMeta {
  int32_t* counter;
  int32_t* slot;
  int32_t* pending;
  int32_t* valid;
};

__device__ __forceinline__ RingMeta ring_meta(int32_t* meta, int B) {
  return RingMeta{meta, meta + B, meta + 2 * B, meta + 3 * B};
}

__device__ __forceinline__ bool selected(const uint8_t* mask, int b) {
  return mask == nullptr || mask[b] != 0;
}

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

// Write the current chunk [B, C, Hkv, D] into its reserved slot. Block (0,0,0) also commits
// the retained-token count at the first write after a reserve; every other block only reads
// slot[], which no block of this launch modifies.
__global__ void __launch_bounds__(256)
k_ring_write(const uint4* __restrict__ k_src, const uint4* __restrict__ v_src,
             uint4* __restrict__ k_store, uint4* __restrict__ v_store, int32_t* meta, int B,
             const uint8_t* mask, int C, int n_slots, int vpr, int32_t* err) {
  RingMeta m = ring_meta(meta, B);
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      if (!selected(mask, b)) continue;
      if (m.slot[b] < 0) {
        report(err, SKV_DEV_RING_UNRESERVED);
        continue;
      }
      if (m.pending[b]) {
        const int c = m.counter[b];
        m.valid[b] = (c < n_slots ? c : n_slots) * C;
        m.pending[b] = 0;
      }
    }
  }
  const int row = blockIdx.x;  // b * C + t
  const int b = row / C;
  const int t = row - b * C;
  if (!selected(mask, b)) return;
  const int s = m.slot[b];
  if (s < 0 || s >= n_slots) return;  // unreserved (reported by block 0) or corrupt metadata
  const bool is_v = blockIdx.y != 0;
  const uint4* src = (is_v ? v_src : k_src) + (int64_t)row * vpr;
  uint4* dst = (is_v ? v_store : k_store) + ((int64_t)b * n_slots * C + (int64_t)s * C + t) * vpr;
  copy_row(src, dst, vpr);
}

// ---------------------------------------------------------------------------------------
// Host launchers (called by api.hip after argument validation)
// ---------------------------------------------------------------------------------------
static dim3 copy_block(int vpr) {
  int threads = vpr >= 256 ? 256 : ((vpr + 63) / 64) * 64;
  return dim3(threads);
}

static dim3 copy_grid(int rows, int tensors, int vpr, int threads) {
  int per_block = threads * kCopyUnroll;
  return dim3(rows, tensors, (vpr + per_block - 1) / per_block);
}

hipError_t launch_write_indexed(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                                const int64_t* index, int64_t start, int B, int n, int cap,
                                int vpr, int32_t* err, hipStream_t s) {
  dim3 blk = copy_block(vpr);
  dim3 grd = copy_grid(B * n, v_cache ? 2 : 1, vpr, blk.x);
  hipLaunchKernelGGL(k_write_indexed, grd, blk, 0, s, (const uint4*)k_src, (const uint4*)v_src,
                     (uint4*)k_cache, (uint4*)v_cache, index, start, n, cap, vpr, err);
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
  dim3 blk = copy_block(vpr);
  dim3 grd = copy_grid(B * C, v_store ? 2 : 1, vpr, blk.x);
  hipLaunchKernelGGL(k_ring_write, grd, blk, 0, s, (const uint4*)k_src, (const uint4*)v_src,
                     (uint4*)k_store, (uint4*)v_store, meta, B, mask, C, n_slots, vpr, err);
  return hipGetLastError();
}

}  // namespace skv
