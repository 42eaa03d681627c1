// Device-resident state of the sink-plus-window ring, shared by the ring kernels.
#pragma once
#include "common.h"

namespace skv {

// Ring metadata: int32 [4][B] = counter, slot, pending, valid (structure of arrays, so
// valid[] is directly the [B] kv_len vector attention reads). counter[b] counts the chunks
// reserved since reset, so the current chunk's chronological id is counter[b] - 1.
struct RingMeta {
  int32_t* counter;
  int32_t* slot;
  int32_t* pending;
  int32_t* valid;
};

__device__ __forceinline__ RingMeta ring_meta(int32_t* meta, int B) {
  return RingMeta{meta, meta + B, meta + 2 * B, meta + 3 * B};
}

// batch-element selection mask: nullptr selects every element
__device__ __forceinline__ bool selected(const uint8_t* mask, int b) {
  return mask == nullptr || mask[b] != 0;
}

// First write after a reserve: the chunk counts as stored from now on (valid covers it).
// Run by one workgroup of a ring-write launch.
__device__ __forceinline__ void ring_commit(RingMeta m, int B, const uint8_t* mask, int C,
                                            int n_slots, int32_t* err) {
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

}  // namespace skv
