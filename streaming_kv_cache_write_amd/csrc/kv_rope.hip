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
// A workgroup takes a block of tb consecutive tokens of one batch element (all heads) and one
// tensor (grid.y: 0 = K, 1 = V). The block is cut into units of (token, head, 8 coordinate
// pairs = 16 elements); each thread issues the loads of 4 units before anything else. The K
// workgroups meanwhile compute the fp64 cosine and sine of every (token, pair) of the block
// once, into LDS, where all heads of the token share them; after one barrier each unit is
// rotated from its registers and stored. V workgroups copy their units unchanged. The kernels
// are HBM-bound like the plain writes (each K and V byte read once and written once).
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

constexpr int kRopeUnits = 4;          // units whose loads a thread issues together
constexpr int kRopeTablePairs = 2048;  // (cos, sin) entries in LDS: 32 KB of fp64

// Token t of the block -> its absolute position and its destination row (element offset of
// the row in the destination tensor); ok = false: the token is not written.
struct RopeTok {
  int64_t pos;
  int64_t dst_row;
  bool ok;
};

#ifndef SKV_ROPE_TRIG_FIRST
#define SKV_ROPE_TRIG_FIRST 1
#endif

// One workgroup: tokens [t0, t0 + nt) of one batch element. src points at token t0's row;
// pos_of(t) gives a block-local token's absolute position (it may read memory), place(p, t)
// its destination and whether it is written (arithmetic only). ROTATE: K (rotate by the
// LDS table), else V (copy). Units: u -> token u / (Hkv*G), head, group g (G = D/16); pairs
// 8g .. 8g+7 are elements (8g + j, D/2 + 8g + j) in layout 0 and (16g + 2j, 16g + 2j + 1) in
// layout 1.
//
// Ordering matters here because the hardware counts outstanding loads in issue order: a wait
// for one load is a wait for every load issued before it. So the frequencies and positions
// the angle table needs are loaded before any unit, and nothing waits on the unit loads until
// their rotation. The source and destination
// pointers carry no restrict qualifier and an empty asm with a memory clobber follows the
// unit loads: otherwise the compiler, seeing loads of read-only memory, moves each unit's
// loads down next to its stores and only one unit's loads are in flight at a time.
template <typename T, int LAYOUT, bool ROTATE, typename PosFn, typename PlaceFn>
__device__ __forceinline__ void rope_block(const T* src, T* dst, int nt, int Hkv, int D,
                                           const double* __restrict__ inv_freq, PosFn pos_of,
                                           PlaceFn place, double2* table, int32_t* err) {
#pragma clang fp contract(off)
  const int G = D / 16, per_tok = Hkv * G, units = nt * per_tok, half = D / 2;
  const int64_t row = (int64_t)Hkv * D;
  const int tid = threadIdx.x;
  constexpr int NI = kRopeTablePairs / kRopeThreads;  // table entries per thread, at most
  double f[NI];
  int64_t kp[NI];
  // the block's angles: entry q = tid + i * kRopeThreads is (token q / half, pair q % half)
  auto angle_inputs = [&]() {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = min(tid + i * kRopeThreads, nt * half - 1);  // clamped: loads unconditional
      const int t = q / half;
      f[i] = inv_freq[q - t * half];
      kp[i] = pos_of(t);
    }
  };
  auto fill_table = [&]() {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = tid + i * kRopeThreads;
      if (q >= nt * half) break;
      double sn = 0.0, cs = 1.0;
      if (place(kp[i], q / half).ok) sincos((double)kp[i] * f[i], &sn, &cs);
      table[q] = make_double2(cs, sn);
    }
    __syncthreads();
  };
  if (ROTATE) {
    angle_inputs();
    if (SKV_ROPE_TRIG_FIRST) fill_table();
  }
  for (int base = 0; base < units; base += kRopeThreads * kRopeUnits) {
    Raw8<T> ru[kRopeUnits], rw[kRopeUnits];
    int ut[kRopeUnits], uh[kRopeUnits], ug[kRopeUnits];
    int64_t up[kRopeUnits];
#pragma unroll
    for (int i = 0; i < kRopeUnits; ++i) {  // each unit's loads go out as soon as its address is known
      const int u = min(base + tid + i * kRopeThreads, units - 1);  // clamped
      ut[i] = u / per_tok;
      const int r = u - ut[i] * per_tok;
      uh[i] = r / G;
      ug[i] = r - uh[i] * G;
      up[i] = pos_of(ut[i]);
      const T* sp = src + ut[i] * row + (int64_t)uh[i] * D;
      ru[i] = ld8(sp + (LAYOUT == 0 ? 8 * ug[i] : 16 * ug[i]));
      rw[i] = ld8(sp + (LAYOUT == 0 ? half + 8 * ug[i] : 16 * ug[i] + 8));
    }
    asm volatile("" ::: "memory");
    if (ROTATE && !SKV_ROPE_TRIG_FIRST && base == 0) fill_table();
#pragma unroll
    for (int i = 0; i < kRopeUnits; ++i) {
      if (base + tid + i * kRopeThreads >= units) break;
      const RopeTok uk = place(up[i], ut[i]);
      if (!uk.ok) {
        if (ROTATE && uh[i] == 0 && ug[i] == 0) report(err, SKV_DEV_INDEX_RANGE);
        continue;
      }
      T* dp = dst + uk.dst_row + (int64_t)uh[i] * D;
      T* d0 = dp + (LAYOUT == 0 ? 8 * ug[i] : 16 * ug[i]);
      T* d1 = dp + (LAYOUT == 0 ? half + 8 * ug[i] : 16 * ug[i] + 8);
      if constexpr (!ROTATE) {
        *(Raw8<T>*)d0 = ru[i];
        *(Raw8<T>*)d1 = rw[i];
      } else {
        double x[8], y[8], a[8], b[8];
        cvt8(ru[i], x);
        cvt8(rw[i], y);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (LAYOUT == 0) {
            a[j] = x[j];
            b[j] = y[j];
          } else {  // elements 16g .. 16g+15 hold pairs (2j, 2j+1)
            a[j] = j < 4 ? x[2 * j] : y[2 * j - 8];
            b[j] = j < 4 ? x[2 * j + 1] : y[2 * j - 7];
          }
        }
        const double2* tp = table + ut[i] * half + 8 * ug[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double2 cs = tp[j];
          const double ac = a[j] * cs.x, bs = b[j] * cs.y, as = a[j] * cs.y, bc = b[j] * cs.x;
          const double ra = ac - bs, rb = as + bc;
          if (LAYOUT == 0) {
            x[j] = ra;
            y[j] = rb;
          } else if (j < 4) {
            x[2 * j] = ra;
            x[2 * j + 1] = rb;
          } else {
            y[2 * j - 8] = ra;
            y[2 * j - 7] = rb;
          }
        }
        store8(d0, x);
        store8(d1, y);
      }
    }
  }
}

// Workgroup -> (batch element, token block, tensor): with V present the K and V workgroups
// of a block alternate, so both kinds are in flight from the start (K workgroups begin with
// their angle table, V workgroups with loads).
struct RopeWg {
  int b, t0, is_v;
};
__device__ __forceinline__ RopeWg rope_wg(int tb, int tblocks, bool has_v) {
  const int nk = has_v ? 2 : 1, wg = blockIdx.x / nk;
  const int b = wg / tblocks;
  return RopeWg{b, (wg - b * tblocks) * tb, (int)blockIdx.x - wg * nk};
}

// Indexed slab write with rotated keys: cache[b, p] = rope(src[b, t], p), p = index[t]
// (IDX false: start + t); rows with p outside [0, cap) are skipped and reported.
// Grid B * tblocks * (1 + has V), tb tokens per workgroup.
template <typename T, int LAYOUT, bool IDX>
__global__ void __launch_bounds__(kRopeThreads)
k_write_indexed_rope(const T* k_src, const T* v_src, T* k_cache, T* v_cache,
                     const int64_t* __restrict__ index, int64_t start, int n, int cap, int Hkv,
                     int D, const double* __restrict__ inv_freq, int tb, int tblocks, int32_t* err) {
  extern __shared__ double2 table[];  // tb * D/2 entries
  const RopeWg w = rope_wg(tb, tblocks, v_src != nullptr);
  const int nt = min(tb, n - w.t0);
  const int64_t row = (int64_t)Hkv * D;
  auto pos_of = [&](int t) -> int64_t { return IDX ? index[w.t0 + t] : start + w.t0 + t; };
  auto place = [&](int64_t p, int) {
    const bool ok = p >= 0 && p < cap;
    return RopeTok{p, ((int64_t)w.b * cap + (ok ? p : 0)) * row, ok};
  };
  const int64_t src_off = ((int64_t)w.b * n + w.t0) * row;
  if (!w.is_v)
    rope_block<T, LAYOUT, true>(k_src + src_off, k_cache, nt, Hkv, D, inv_freq, pos_of, place, table, err);
  else
    rope_block<T, LAYOUT, false>(v_src + src_off, v_cache, nt, Hkv, D, inv_freq, pos_of, place, table, err);
}

// Ring write with rotated keys: the chunk of batch element b goes to its reserved slot; row t
// is rotated at position (counter[b] - 1) * C + t. Grid B * tblocks * (1 + has V).
template <typename T, int LAYOUT>
__global__ void __launch_bounds__(kRopeThreads)
k_ring_write_rope(const T* k_src, const T* v_src, T* k_store, T* v_store, int32_t* meta, int B,
                  const uint8_t* mask, int C, int n_slots, int Hkv, int D,
                  const double* __restrict__ inv_freq, int tb, int tblocks, int32_t* err) {
  extern __shared__ double2 table[];  // tb * D/2 entries
  RingMeta m = ring_meta(meta, B);
  if (blockIdx.x == 0) ring_commit(m, B, mask, C, n_slots, err);
  const RopeWg w = rope_wg(tb, tblocks, v_src != nullptr);
  if (!selected(mask, w.b)) return;
  const int slot = m.slot[w.b];
  if (slot < 0 || slot >= n_slots) return;  // unreserved (reported by workgroup 0) or corrupt
  const int nt = min(tb, C - w.t0);
  const int64_t row = (int64_t)Hkv * D;
  const int64_t pos0 = (int64_t)(m.counter[w.b] - 1) * C + w.t0;
  const int64_t dst0 = (((int64_t)w.b * n_slots + slot) * C + w.t0) * row;
  auto pos_of = [&](int t) -> int64_t { return pos0 + t; };
  auto place = [&](int64_t p, int t) { return RopeTok{p, dst0 + t * row, true}; };
  const int64_t src_off = ((int64_t)w.b * C + w.t0) * row;
  if (!w.is_v)
    rope_block<T, LAYOUT, true>(k_src + src_off, k_store, nt, Hkv, D, inv_freq, pos_of, place, table, err);
  else
    rope_block<T, LAYOUT, false>(v_src + src_off, v_store, nt, Hkv, D, inv_freq, pos_of, place, table, err);
}

// Tokens per workgroup: about kRopeThreads * kRopeUnits units, at most what the LDS table holds
static int rope_tokens_per_block(int Hkv, int D) {
  const int per_tok = Hkv * (D / 16);
  int tb = (kRopeThreads * kRopeUnits) / per_tok;
  if (tb < 1) tb = 1;
  const int cap = kRopeTablePairs / (D / 2);
  return tb < cap ? tb : cap;
}

static size_t rope_table_bytes(int tb, int D) { return (size_t)tb * (D / 2) * sizeof(double2); }

template <typename T, int LAYOUT>
static hipError_t write_indexed_rope_t(const void* k_src, const void* v_src, void* k_cache,
                                       void* v_cache, const int64_t* index, int64_t start, int B,
                                       int n, int cap, int Hkv, int D, const double* inv_freq,
                                       int32_t* err, hipStream_t s) {
  const int tb = rope_tokens_per_block(Hkv, D);
  const int tblocks = (n + tb - 1) / tb;
  dim3 grd((unsigned)((int64_t)B * tblocks * (v_src ? 2 : 1)));
  if (index)
    hipLaunchKernelGGL((k_write_indexed_rope<T, LAYOUT, true>), grd, dim3(kRopeThreads),
                       rope_table_bytes(tb, D), s, (const T*)k_src, (const T*)v_src, (T*)k_cache,
                       (T*)v_cache, index, start, n, cap, Hkv, D, inv_freq, tb, tblocks, err);
  else
    hipLaunchKernelGGL((k_write_indexed_rope<T, LAYOUT, false>), grd, dim3(kRopeThreads),
                       rope_table_bytes(tb, D), s, (const T*)k_src, (const T*)v_src, (T*)k_cache,
                       (T*)v_cache, index, start, n, cap, Hkv, D, inv_freq, tb, tblocks, err);
  return hipGetLastError();
}

template <typename T, int LAYOUT>
static hipError_t ring_write_rope_t(const void* k_src, const void* v_src, void* k_store,
                                    void* v_store, int32_t* meta, int B, const uint8_t* mask,
                                    int C, int n_slots, int Hkv, int D, const double* inv_freq,
                                    int32_t* err, hipStream_t s) {
  const int tb = rope_tokens_per_block(Hkv, D);
  const int tblocks = (C + tb - 1) / tb;
  dim3 grd((unsigned)((int64_t)B * tblocks * (v_src ? 2 : 1)));
  hipLaunchKernelGGL((k_ring_write_rope<T, LAYOUT>), grd, dim3(kRopeThreads), rope_table_bytes(tb, D), s,
                     (const T*)k_src, (const T*)v_src, (T*)k_store, (T*)v_store, meta, B, mask, C,
                     n_slots, Hkv, D, inv_freq, tb, tblocks, err);
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
