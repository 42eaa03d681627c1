// Device-side helpers shared by the libskv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/skv.h"

namespace skv {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

__device__ __forceinline__ void report(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int bytes = 4; };
template <> struct Elem<bf16_t> { static constexpr int bytes = 2; };
template <> struct Elem<f16_t> { static constexpr int bytes = 2; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }

// Attention workspace: its first kWsCounterInts int32 are arrival counters, which every launch
// leaves at zero; partials follow. The counter area has the same size for every kernel that
// takes a workspace, so one workspace of the largest size needed can serve any sequence of
// calls: no call's counters ever overlap another call's partials.
constexpr int kWsCounterInts = 16384;  // 64 KiB

// Which keys batch element b attends to, read from the device metadata at run time.
//   prefix mode: rows [0, len) of the batch element's cap-row slab; with the full-capacity
//                arm all cap rows are visited and rows >= len are masked.
//   packed mode: rows [cu[b], cu[b+1]) of the packed buffer.
struct KeySet {
  int64_t base_row;  // first row of this batch element in the K/V buffer
  int len;           // active keys (kv_len or segment length)
  int visit;         // rows the kernel iterates over (len, or cap for the full-capacity arm)
  bool ok;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* kv_len_dev;
  const int32_t* cu;
  int32_t* err;
  int B, Tq, Hq, Hkv, cap, kv_len_host;
  int mask, block;
  int full_cap;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  // fused decode step only: new rows [B, Tq, Hkv, D], the shared write cursor, kv_len output
  const void* k_new;
  const void* v_new;
  int32_t* cursor;
  int32_t* kv_len_out;
};

// Metadata the kernels only read, through the constant address space: uniform reads of it
// are then always scalar loads (with the vector loads of the same launch in flight, a vector
// load of a length would have to wait for all of them).
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int read_meta(const int32_t* p, int i) {
  return ((const_i32*)p)[i];
}

__device__ __forceinline__ KeySet key_set(const AttnArgs& a, int b) {
  KeySet s;
  if (a.cu) {
    int lo = read_meta(a.cu, b), hi = read_meta(a.cu, b + 1);
    // cap is the packed buffer's row count here: a segment may not run past it
    bool ok = (b > 0 || lo == 0) && hi > lo && hi <= a.cap;
    s.base_row = lo;
    s.len = ok ? hi - lo : 0;
    s.visit = s.len;
    s.ok = ok;
  } else {
    int len = a.kv_len_dev ? read_meta(a.kv_len_dev, b) : a.kv_len_host;
    bool ok = len >= 1 && len <= a.cap;
    s.base_row = (int64_t)b * a.cap;
    s.len = ok ? len : 0;
    s.visit = ok ? (a.full_cap ? a.cap : len) : 0;
    s.ok = ok;
  }
  // a causal chunk longer than the prefix would leave its first queries without keys
  if (s.ok && a.mask != SKV_MASK_NONE && a.Tq > s.len) s.ok = false;
  return s;
}

__device__ __forceinline__ int dev_error_bit(const AttnArgs& a) {
  return a.cu ? SKV_DEV_CU_SEQLENS : SKV_DEV_KV_LEN;
}

// Largest key index a query at absolute position p may see under the mask (queries are
// bottom-right aligned: query t of Tq sits at p = len - Tq + t). Key j is visible iff
// j <= min(mask_limit(p), len - 1). CAUSAL is BLOCK_CAUSAL with block 1. Computed once per
// query row, so the per-score test is a single compare-and-select with no branch.
__device__ __forceinline__ int mask_limit(int mask, int block, int p) {
  if (mask == SKV_MASK_NONE) return 0x7fffffff;
  return (p / block + 1) * block - 1;  // p >= 0 whenever a mask is set (checked by key_set)
}

__device__ __forceinline__ int row_limit(int mask, int block, int p, int len) {
  const int m = mask_limit(mask, block, p);
  return m < len - 1 ? m : len - 1;
}

}  // namespace skv
