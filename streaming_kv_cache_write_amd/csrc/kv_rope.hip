// Cache writes that rotate each key at its absolute position on the way in: the rotary
// embedding fused into the indexed slab write and into the ring write, so K is read and
// written once instead of twice (a separate rotation pass, then the copy).
//
// flashdreams issue #763 "add an opt-in circular KV policy for streaming attention", section
// proposed boundary: keys are rotated at their absolute positions before the cache write, which
// is what lets a circular buffer keep them in physical order. The page gives no formula; the
// reading implemented here: coordinate pairs (a, b) of a key row -- (i, i + D/2) or (2i, 2i+1)
// -- turn by theta = position * inv_freq[i], (a, b) -> (a cos - b sin, a sin + b cos), with the
// caller's frequency table, in fp64 (angle, sine, cosine, products and sums, no fused
// multiply-add), rounded to fp32 and then to the cache type (round to nearest even). A key's
// position is its slab row (the write index), or chunk_id * C + t in the ring (chunk_id = the
// number of chunks reserved before it since reset). V rows are copied unchanged.
//
// One thread takes one token row and 8 coordinate pairs (16 elements) of every head: the 8
// sines and cosines are computed once and reused for all Hkv heads, whose loads go out four
// heads at a time. The kernels are HBM-bound like the plain writes (each K and V byte read
// once and written once); the fp64 trig costs 8 sincos per (token, 8 pairs), not per head.
#include "common.h"
#include "ring_meta.h"

namespace skv {

constexpr int kRopeThreads = 256;

// 8 consecutive elements as raw 16-byte vectors, and their exact fp64 values
template <typename T> struct Raw8 { i32x4 v[sizeof(T) / 2]; };
template <typename T>
__device__ __forceinline__ Raw8<T> ld8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)sizeof(T) / 2; ++i) r.v[i] = ((const i32x4*)p)[i];
  return r;
}
__device__ __forceinline__ void cvt8(const Raw8<bf16_t>& r, double* x) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, r.v[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (double)(float)v[j];
}
__device__ __forceinline__ void cvt8(const Raw8<f16_t>& r, double* x) {
  const f16x8 v = __builtin_bit_cast(f16x8, r.v[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (double)(float)v[j];
}
__device__ __forceinline__ void cvt8(const Raw8<float>& r, double* x) {
  const f32x4 u = __builtin_bit_cast(f32x4, r.v[0]), w = __builtin_bit_cast(f32x4, r.v[1]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = u[j];
    x[4 + j] = w[j];
  }
}
// fp64 -> fp32 (round to nearest even) -> cache type (round to nearest even). Left alone, the
// compiler folds the two conversions into one direct fp64 -> fp16 rounding, which differs
// whenever the fp32 step lands exactly on an fp16 halfway point; the empty asm keeps the
// fp32 value as an operand of its own.
__device__ __forceinline__ float to_f32_rne(double x) {
  float f = (float)x;
  asm volatile("" : "+v"(f));
  return f;
}
__device__ __forceinline__ void store8(bf16_t* p, const double* x) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16_t)to_f32_rne(x[j]);
  *(bf16x8*)p = v;
}
__device__ __forceinline__ void store8(f16_t* p, const double* x) {
  f16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (f16_t)to_f32_rne(x[j]);
  *(f16x8*)p = v;
}
__device__ __forceinline__ void store8(float* p, const double* x) {
  *(float4*)p = make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  *(float4*)(p + 4) = make_float4((float)x[4], (float)x[5], (float)x[6], (float)x[7]);
}

// cos and sin of position * inv_freq[8g + j], j < 8
__device__ __forceinline__ void rope_angles(int64_t pos, const double* inv_freq, int g, double* c,
                                            double* s) {
#pragma unroll
  for (int j = 0; j < 8; ++j) sincos((double)pos * inv_freq[8 * g + j], &s[j], &c[j]);
}

constexpr int kRopeHeadGroup = 4;  // heads whose loads are issued together

// Rotate pairs 8g .. 8g+7 of every head of one token row at position pos. LAYOUT 0: pair
// i = (i, i + D/2); LAYOUT 1: pair i = (2i, 2i + 1). Heads go in groups of kRopeHeadGroup,
// alternating between two register buffers: the next group's loads are in flight while a
// group is rotated and stored (the first group's also while the angles are computed).
template <typename T, int LAYOUT>
__device__ __forceinline__ void rope_row(const T* src, T* dst, int Hkv, int D, int g, int64_t pos,
                                         const double* inv_freq) {
#pragma clang fp contract(off)
  constexpr int HB = kRopeHeadGroup;
  const int o0 = LAYOUT == 0 ? 8 * g : 16 * g;
  const int o1 = LAYOUT == 0 ? D / 2 + 8 * g : 16 * g + 8;
  Raw8<T> bu[2][HB], bw[2][HB];
  auto load_group = [&](int buf, int h0) {
#pragma unroll
    for (int k = 0; k < HB; ++k)
      if (h0 + k < Hkv) {
        bu[buf][k] = ld8(src + (int64_t)(h0 + k) * D + o0);
        bw[buf][k] = ld8(src + (int64_t)(h0 + k) * D + o1);
      }
  };
  load_group(0, 0);
  double c[8], s[8];
  rope_angles(pos, inv_freq, g, c, s);
  auto rotate_group = [&](int buf, int h0) {
#pragma unroll
    for (int k = 0; k < HB; ++k) {
      if (h0 + k >= Hkv) break;
      double u[8], w[8], a[8], b[8];
      cvt8(bu[buf][k], u);
      cvt8(bw[buf][k], w);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (LAYOUT == 0) {
          a[j] = u[j];
          b[j] = w[j];
        } else {  // elements 16g .. 16g+15 hold pairs (2j, 2j+1)
          a[j] = j < 4 ? u[2 * j] : w[2 * j - 8];
          b[j] = j < 4 ? u[2 * j + 1] : w[2 * j - 7];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double ac = a[j] * c[j], bs = b[j] * s[j], as = a[j] * s[j], bc = b[j] * c[j];
        const double ra = ac - bs, rb = as + bc;
        if (LAYOUT == 0) {
          u[j] = ra;
          w[j] = rb;
        } else if (j < 4) {
          u[2 * j] = ra;
          u[2 * j + 1] = rb;
        } else {
          w[2 * j - 8] = ra;
          w[2 * j - 7] = rb;
        }
      }
      T* dp = dst + (int64_t)(h0 + k) * D;
      store8(dp + o0, u);
      store8(dp + o1, w);
    }
  };
  for (int h0 = 0; h0 < Hkv; h0 += 2 * HB) {
    load_group(1, h0 + HB);
    rotate_group(0, h0);
    load_group(0, h0 + 2 * HB);
    rotate_group(1, h0 + HB);
  }
}

// The same 16 elements of every head, copied (V rows)
template <typename T>
__device__ __forceinline__ void copy_row(const T* src, T* dst, int Hkv, int D, int g) {
  constexpr int V = 16 * sizeof(T) / 16;  // 16-byte vectors per 16 elements
#pragma unroll 2
  for (int h = 0; h < Hkv; ++h) {
    const i32x4* sp = (const i32x4*)(src + (int64_t)h * D + 16 * g);
    i32x4* dp = (i32x4*)(dst + (int64_t)h * D + 16 * g);
    i32x4 r[V];
#pragma unroll
    for (int v = 0; v < V; ++v) r[v] = __builtin_nontemporal_load(sp + v);
#pragma unroll
    for (int v = 0; v < V; ++v) dp[v] = r[v];
  }
}

// Indexed slab write with rotated keys: cache[b, p] = rope(src[b, t], p), p = index[t]
// (index == nullptr: start + t). Grid (B * tblocks, 1 + has V); thread -> (token t, group g).
template <typename T, int LAYOUT>
__global__ void __launch_bounds__(kRopeThreads)
k_write_indexed_rope(const T* __restrict__ k_src, const T* __restrict__ v_src,
                     T* __restrict__ k_cache, T* __restrict__ v_cache,
                     const int64_t* __restrict__ index, int64_t start, int n, int cap, int Hkv,
                     int D, const double* __restrict__ inv_freq, int tblocks, int32_t* err) {
  const int gpt = D / 16, tpb = kRopeThreads / gpt;
  const int b = blockIdx.x / tblocks, tb = blockIdx.x - b * tblocks;
  const int t = tb * tpb + (int)threadIdx.x / gpt, g = (int)threadIdx.x % gpt;
  if (t >= n) return;
  const int64_t pos = index ? index[t] : start + t;
  const bool is_v = blockIdx.y != 0;
  if (pos < 0 || pos >= cap) {
    if (!is_v && g == 0) report(err, SKV_DEV_INDEX_RANGE);
    return;
  }
  const int64_t row = (int64_t)Hkv * D;
  if (is_v) {
    copy_row<T>(v_src + ((int64_t)b * n + t) * row, v_cache + ((int64_t)b * cap + pos) * row, Hkv, D, g);
    return;
  }
  rope_row<T, LAYOUT>(k_src + ((int64_t)b * n + t) * row, k_cache + ((int64_t)b * cap + pos) * row,
                      Hkv, D, g, pos, inv_freq);
}

// Ring write with rotated keys: the chunk of batch element b goes to its reserved slot; row t
// is rotated at position (counter[b] - 1) * C + t. Grid (B * tblocks, 1 + has V).
template <typename T, int LAYOUT>
__global__ void __launch_bounds__(kRopeThreads)
k_ring_write_rope(const T* __restrict__ k_src, const T* __restrict__ v_src,
                  T* __restrict__ k_store, T* __restrict__ v_store, int32_t* meta, int B,
                  const uint8_t* mask, int C, int n_slots, int Hkv, int D,
                  const double* __restrict__ inv_freq, int tblocks, int32_t* err) {
  RingMeta m = ring_meta(meta, B);
  if (blockIdx.x == 0 && blockIdx.y == 0) ring_commit(m, B, mask, C, n_slots, err);
  const int gpt = D / 16, tpb = kRopeThreads / gpt;
  const int b = blockIdx.x / tblocks, tb = blockIdx.x - b * tblocks;
  const int t = tb * tpb + (int)threadIdx.x / gpt, g = (int)threadIdx.x % gpt;
  if (t >= C || !selected(mask, b)) return;
  const int slot = m.slot[b];
  if (slot < 0 || slot >= n_slots) return;  // unreserved (reported by workgroup 0) or corrupt
  const int64_t row = (int64_t)Hkv * D;
  const int64_t src_off = ((int64_t)b * C + t) * row;
  const int64_t dst_off = (((int64_t)b * n_slots + slot) * C + t) * row;
  if (blockIdx.y != 0) {
    copy_row<T>(v_src + src_off, v_store + dst_off, Hkv, D, g);
    return;
  }
  rope_row<T, LAYOUT>(k_src + src_off, k_store + dst_off, Hkv, D, g,
                      (int64_t)(m.counter[b] - 1) * C + t, inv_freq);
}

template <typename T, int LAYOUT>
static hipError_t write_indexed_rope_t(const void* k_src, const void* v_src, void* k_cache,
                                       void* v_cache, const int64_t* index, int64_t start, int B,
                                       int n, int cap, int Hkv, int D, const double* inv_freq,
                                       int32_t* err, hipStream_t s) {
  const int tpb = kRopeThreads / (D / 16);
  const int tblocks = (n + tpb - 1) / tpb;
  dim3 grd((unsigned)((int64_t)B * tblocks), v_src ? 2 : 1);
  hipLaunchKernelGGL((k_write_indexed_rope<T, LAYOUT>), grd, dim3(kRopeThreads), 0, s,
                     (const T*)k_src, (const T*)v_src, (T*)k_cache, (T*)v_cache, index, start, n,
                     cap, Hkv, D, inv_freq, tblocks, err);
  return hipGetLastError();
}

template <typename T, int LAYOUT>
static hipError_t ring_write_rope_t(const void* k_src, const void* v_src, void* k_store,
                                    void* v_store, int32_t* meta, int B, const uint8_t* mask,
                                    int C, int n_slots, int Hkv, int D, const double* inv_freq,
                                    int32_t* err, hipStream_t s) {
  const int tpb = kRopeThreads / (D / 16);
  const int tblocks = (C + tpb - 1) / tpb;
  dim3 grd((unsigned)((int64_t)B * tblocks), v_src ? 2 : 1);
  hipLaunchKernelGGL((k_ring_write_rope<T, LAYOUT>), grd, dim3(kRopeThreads), 0, s,
                     (const T*)k_src, (const T*)v_src, (T*)k_store, (T*)v_store, meta, B, mask, C,
                     n_slots, Hkv, D, inv_freq, tblocks, err);
  return hipGetLastError();
}

// Host-checked before these are called: D a power of two in [16, 4096], dtype known,
// layout 0 or 1, B * tblocks within the grid limit.
hipError_t launch_write_indexed_rope(const void* k_src, const void* v_src, void* k_cache,
                                     void* v_cache, const int64_t* index, int64_t start, int B,
                                     int n, int cap, int Hkv, int D, int dtype,
                                     const double* inv_freq, int layout, int32_t* err,
                                     hipStream_t s) {
#define SKV_ROPE_W(T, L) \
  write_indexed_rope_t<T, L>(k_src, v_src, k_cache, v_cache, index, start, B, n, cap, Hkv, D, inv_freq, err, s)
  if (dtype == SKV_BF16) return layout ? SKV_ROPE_W(bf16_t, 1) : SKV_ROPE_W(bf16_t, 0);
  if (dtype == SKV_F16) return layout ? SKV_ROPE_W(f16_t, 1) : SKV_ROPE_W(f16_t, 0);
  return layout ? SKV_ROPE_W(float, 1) : SKV_ROPE_W(float, 0);
#undef SKV_ROPE_W
}

hipError_t launch_ring_write_rope(const void* k_src, const void* v_src, void* k_store,
                                  void* v_store, int32_t* meta, int B, const uint8_t* mask, int C,
                                  int n_slots, int Hkv, int D, int dtype, const double* inv_freq,
                                  int layout, int32_t* err, hipStream_t s) {
#define SKV_ROPE_R(T, L) \
  ring_write_rope_t<T, L>(k_src, v_src, k_store, v_store, meta, B, mask, C, n_slots, Hkv, D, inv_freq, err, s)
  if (dtype == SKV_BF16) return layout ? SKV_ROPE_R(bf16_t, 1) : SKV_ROPE_R(bf16_t, 0);
  if (dtype == SKV_F16) return layout ? SKV_ROPE_R(f16_t, 1) : SKV_ROPE_R(f16_t, 0);
  return layout ? SKV_ROPE_R(float, 1) : SKV_ROPE_R(float, 0);
#undef SKV_ROPE_R
}

}  // namespace skv
