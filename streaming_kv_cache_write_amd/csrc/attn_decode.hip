// Decode-sized attention (Tq <= 4, Tq * Hq/Hkv <= 16 query rows per KV head): split-K over the
// key range with the LSE-weighted merge of the splits done in the same launch.
//
// Each decode step i attends its single new query to the active prefix kv_len = T + i + 1
// (fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA",
// section Change). A step reads 2*kv_len*Hkv*D*elem bytes of K/V and does little math per
// byte; at the lengths of a decode job it is bound by the chain of dependent steps (cursor ->
// loads -> math -> merge), so the kernel keeps that chain short and spreads the loads over
// many CUs:
//   * one workgroup of 4 wavefronts per (split, KV head g, batch element b); the split's key
//     range is dealt out to the wavefronts in 16-key tiles, and each wavefront keeps the loads
//     of its next two tiles in flight while it works on the current one;
//   * the query rows of a GQA group (R = Tq * Hq/Hkv <= 16, padded to 16) share each K/V load.
//     S^T = K Q^T runs on v_mfma_f32_16x16x32 with K straight from global memory as the A
//     operand; its accumulator leaves, in each lane, four keys of one query row -- exactly the
//     A-operand layout of v_mfma_f32_16x16x16, so P V runs on the matrix cores with P staying
//     in the lane that computed it. V^T operands come from a small per-wavefront LDS tile by
//     transposed reads (ds_read_b64_tr_b16);
//   * online softmax in fp32 with exp2 (scale folded), the row max over a tile by two
//     cross-lane exchanges; the reference max moves only when a tile's max passes it by more
//     than 2^8 in probability (the stale reference cancels in O / l);
//   * the 4 wavefronts merge through LDS, one thread per (row quad, column); with several
//     splits each workgroup stores its unnormalised (m, l, o) to the caller's workspace with
//     device-coherent (sc1) stores -- the form agent-scope atomic stores take, visible to any
//     XCD once complete -- and counts itself in; the last workgroup of (b, g) to arrive reads
//     them back with sc1 loads, first every split's weight exp(m_s - max m) / L (one
//     half-wavefront per row, DPP reductions), then one weighted pass over the o partials,
//     whose loads are already in flight, and writes the output.
#include <type_traits>

#include "common.h"

namespace skv {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short dec_s16x4;
typedef __attribute__((address_space(3))) dec_s16x4 dec_lds_s16x4;

template <typename T> struct DecMma;
template <> struct DecMma<bf16_t> {
  typedef bf16x8 vec8;
  typedef dec_s16x4 vec4;
  static __device__ __forceinline__ f32x4 qk(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 pack(float x0, float x1, float x2, float x3) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 b4;
    const b4 v = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
    return __builtin_bit_cast(vec4, v);
  }
  // running sum plus the four rounded values (two dot2 with (1, 1))
  static __device__ __forceinline__ float sum4(vec4 p, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 b2;
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 b4;
    const b4 v = __builtin_bit_cast(b4, p);
    const b2 one = {(__bf16)1.f, (__bf16)1.f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(b2{v[0], v[1]}, one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(b2{v[2], v[3]}, one, acc, false);
  }
};
template <> struct DecMma<f16_t> {
  typedef f16x8 vec8;
  typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 vec4;
  static __device__ __forceinline__ f32x4 qk(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 pack(float x0, float x1, float x2, float x3) {
    return vec4{(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
  }
  static __device__ __forceinline__ float sum4(vec4 p, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2;
    const h2 one = {(_Float16)1.f, (_Float16)1.f};
    acc = __builtin_amdgcn_fdot2(h2{p[0], p[1]}, one, acc, false);
    return __builtin_amdgcn_fdot2(h2{p[2], p[3]}, one, acc, false);
  }
};

constexpr int kDecTile = 16;    // keys per wavefront tile (one MFMA block of keys)
constexpr int kDecRows = 16;    // query rows per KV head (MFMA block; R <= 16 are used)
// Workgroup shape: W wavefronts take W tiles (a chunk of 16 W keys) per round.
template <int W> struct DecShape {
  static constexpr int waves = W, chunk = kDecTile * W, threads = 64 * W;
};
constexpr int kDecWaves = 4;
constexpr int kDecMaxSplits = 32;
constexpr float kDecRescaleLog2 = 8.f;

// the shared counter area: B*Hkv split counters + 1 (host-checked to fit)
__host__ __device__ __forceinline__ size_t dec_counter_floats(int, int) { return kWsCounterInts; }
__host__ __device__ __forceinline__ size_t dec_o_floats(int B, int Hkv, int D, int n_splits) {
  return (size_t)B * Hkv * n_splits * kDecRows * D;
}
__host__ __device__ __forceinline__ size_t dec_ml_floats(int B, int Hkv, int n_splits) {
  return ((size_t)B * Hkv * n_splits * kDecRows * 2 + 3) & ~(size_t)3;  // keep 16-byte alignment
}

// Split partials cross XCDs, whose L2 caches are not coherent with each other. They are
// stored and loaded with the sc1 cache policy -- device-coherent, as agent-scope atomic
// stores and loads are -- so a store that has completed (vmcnt drained) is visible to a later
// sc1 load from any CU, with no cache write-back or invalidate.
constexpr int kDeviceCoherent = 16;  // buffer-op cache policy bits: sc1
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0)
// s_waitcnt vmcnt(2 * LT) (gfx9 encoding: vmcnt low bits 3:0, high bits 15:14; expcnt and
// lgkmcnt at their maxima)
template <int LT> constexpr int kWaitVmcntTwoTiles() {
  static_assert(2 * LT < 64, "vmcnt field");
  return (0x0F70 & ~0xC00F) | ((2 * LT) & 0xF) | (((2 * LT) >> 4) << 14);
}
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float* base, size_t floats) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(floats * sizeof(float)),
                                           0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, size_t fidx, float4 v) {
  const u32x4 d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                   __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, (int)(fidx * sizeof(float)), 0, kDeviceCoherent);
}
__device__ __forceinline__ float4 load_coherent4(__amdgpu_buffer_rsrc_t r, size_t fidx) {
  const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(fidx * sizeof(float)), 0, kDeviceCoherent);
  return make_float4(__uint_as_float(d[0]), __uint_as_float(d[1]), __uint_as_float(d[2]),
                     __uint_as_float(d[3]));
}

// Partial layout: split `split` of (b, g) holds o as [4 row quads][D] float4 (rows 4q .. 4q+3
// of one column in one float4), then (m, l) as 16 maxima followed by 16 sums.
__device__ __forceinline__ size_t dec_o_quad(int b, int g, int split, int rq, int Hkv,
                                             int n_splits, int D) {
  return ((((size_t)b * Hkv + g) * n_splits + split) * 4 + rq) * D;  // in float4 units
}
__device__ __forceinline__ size_t dec_ml_base(int b, int g, int split, int Hkv, int n_splits) {
  return (((size_t)b * Hkv + g) * n_splits + split) * (2 * kDecRows);
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t r, size_t fidx) {
  return __uint_as_float(
      __builtin_amdgcn_raw_buffer_load_b32(r, (int)(fidx * sizeof(float)), 0, kDeviceCoherent));
}

// Lane exchanges by DPP (every lane of the wavefront active): quad xor 1 and 2, and the two
// mirrors, which with the quad steps reduce over each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// Exchanges with lane ^ 16 and lane ^ 32 by permlane swaps (VALU, no LDS round trip): with
// both operands x, the swap returns the two rows (or halves) of each pair, in either order.
__device__ __forceinline__ float max_xor16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float max32(float x) {  // over each 32-lane half of the wavefront
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  return max_xor16(x);
}
__device__ __forceinline__ float sum32(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return sum_xor16(x);
}

__device__ __forceinline__ float f4_get(float4 v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Output rows 4rq .. 4rq+3 (those < R) at column col; row r = t * group + hh is query t of
// head g * group + hh. v holds the normalised values.
template <typename OutT>
__device__ __forceinline__ void write_quad(const AttnArgs& a, int D, int group, int b, int g,
                                           int rq, int col, float4 v) {
  const int R = a.Tq * group;
  int t = (4 * rq) / group, hh = 4 * rq - t * group;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * rq + j < R)
      ((OutT*)a.out)[(((int64_t)b * a.Tq + t) * a.Hq + g * group + hh) * D + col] =
          from_f32<OutT>(f4_get(v, j));
    if (++hh == group) {
      hh = 0;
      ++t;
    }
  }
}
__device__ __forceinline__ void write_lse(const AttnArgs& a, int group, int b, int g, int r,
                                          float M, float L) {
  const int t = r / group, h = g * group + (r - t * group);
  a.lse[((int64_t)b * a.Hq + h) * a.Tq + t] = L > 0.f ? M * a.scale + logf(L) : -INFINITY;
}

// The last workgroup of (b, g): merge the n_active partials. Every load is unconditional
// (indices clamped, invalid entries neutralised afterwards), so no load waits on a branch. The
// (m, l) loads go first, then the first batch of o loads; step 1 -- thread (row r, split s),
// 32 splits per half-wavefront -- reduces over the splits to the weight exp2((m_s - M) c2) / L
// of each partial (L = the weighted sum of the l_s), kept in LDS, while the o loads are in
// flight. Step 2: thread (row quad, column, split residue mod tpp) sums its splits' weighted
// o; the tpp threads of a pair are adjacent lanes and add by DPP.
template <int D, typename OutT, int NT>
__device__ __forceinline__ void merge_splits(const AttnArgs& a, int group, int RQ, const float* o_bg,
                                             __amdgpu_buffer_rsrc_t rml, float (*wt)[kDecRows], int b,
                                             int g, int n_active, int n_splits) {
  const __amdgpu_buffer_rsrc_t ro_bg = ws_rsrc(o_bg, (size_t)n_active * 4 * D * 4);
  constexpr int kMB = 16;  // o loads in flight per thread
  const int R = a.Tq * group, rows = 4 * RQ;
  const float c2 = a.scale_log2;
  constexpr int NQ = (kDecRows * 32 + NT - 1) / NT;  // (row, split) rounds
  const int pairs = RQ * D;  // (row quad, column)
  const int tpp = 4 * pairs <= NT ? 4 : 2 * pairs <= NT ? 2 : 1;
  const int t = threadIdx.x, sub = t & (tpp - 1), p0 = t / tpp;
  const int p_step = NT / tpp;
  const int last_split = n_active - 1;

  float mm[NQ], ll[NQ];  // (m, l) of (row q / 32, split q % 32) for q = t + NT k
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = t + NT * k;
    const size_t base = dec_ml_base(b, g, min(q & 31, last_split), a.Hkv, n_splits);
    const int r = min(q >> 5, rows - 1);
    mm[k] = load_coherent1(rml, base + r);
    ll[k] = load_coherent1(rml, base + kDecRows + r);
  }
  // o partials of this (b, g) through a resource that ends after the active splits: a load of a
  // split past them returns zeros and moves no data
  float4 ob[kMB];
  auto load_batch = [&](int p, int s0) {
    const int pc = min(p, pairs - 1);
    const int rq = pc / D, col = pc - rq * D;
#pragma unroll
    for (int i = 0; i < kMB; ++i)
      ob[i] = load_coherent4(ro_bg, ((size_t)((s0 + i * tpp) * 4 + rq) * D + col) * 4);
  };
  load_batch(p0, sub);

#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = t + NT * k, r = q >> 5, sp = q & 31;
    const bool ok = r < rows && sp < n_active;
    // a clamped split index repeats the row's last split, which leaves the max unchanged;
    // it gets weight 0 (its l, a finite partial of this launch, then adds nothing)
    const float M = max32(mm[k]);
    const float e = __builtin_amdgcn_exp2f((mm[k] - (M == -INFINITY ? 0.f : M)) * c2);
    const float w = ok ? e : 0.f;
    const float L = sum32(w * ll[k]);
    if (ok) wt[sp][r] = L > 0.f ? w / L : 0.f;
    if (ok && sp == 0 && r < R && a.lse) write_lse(a, group, b, g, r, M, L);
  }
  __syncthreads();

  for (int p = p0; p - p0 < pairs; p += p_step) {  // the same trip count in every thread
    const int pc = min(p, pairs - 1);
    const int rq = pc / D, col = pc - rq * D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = sub; s0 < n_active; s0 += kMB * tpp) {
      if (p != p0 || s0 != sub) load_batch(p, s0);
      float4 w4[kMB];
#pragma unroll
      for (int i = 0; i < kMB; ++i) w4[i] = *(const float4*)&wt[min(s0 + i * tpp, last_split)][4 * rq];
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
        const bool ok = s0 + i * tpp < n_active;
        acc = make_float4(fmaf(ok ? w4[i].x : 0.f, ob[i].x, acc.x), fmaf(ok ? w4[i].y : 0.f, ob[i].y, acc.y),
                          fmaf(ok ? w4[i].z : 0.f, ob[i].z, acc.z), fmaf(ok ? w4[i].w : 0.f, ob[i].w, acc.w));
      }
    }
    if (tpp > 1) {
      acc.x += dpp_f<kDppXor1>(acc.x);
      acc.y += dpp_f<kDppXor1>(acc.y);
      acc.z += dpp_f<kDppXor1>(acc.z);
      acc.w += dpp_f<kDppXor1>(acc.w);
    }
    if (tpp > 2) {
      acc.x += dpp_f<kDppXor2>(acc.x);
      acc.y += dpp_f<kDppXor2>(acc.y);
      acc.z += dpp_f<kDppXor2>(acc.z);
      acc.w += dpp_f<kDppXor2>(acc.w);
    }
    if (sub == 0 && p < pairs) write_quad<OutT>(a, D, group, b, g, rq, col, acc);
  }
}

// Workgroup = W wavefronts per (split, KV head g, batch element b). The split covers whole
// chunks (16 W keys) of the visited range; wavefront w takes the 16-key tiles at offsets 16w,
// 16w + 16W, ... of it. Splits past the last one holding keys leave at once: they store no
// partial and are not waited for, so the merge reads only the splits that did work.
// FUSED: one launch per decode step with the write cursor on the device (attn_decode_step):
// c = *cursor; the new rows k_new/v_new [B, Tq, Hkv, D] are written to cache rows c .. c+Tq-1
// and attended over as keys c .. c+Tq-1 straight from the sources (no wavefront of this launch
// reads a cache row another one writes). Every workgroup counts itself in once it has read the
// cursor; the last one to do so sets *cursor = c+Tq and kv_len_out[:] = c+Tq.
// SPEC: the first tiles of every wavefront are known before the length is read -- each split
// holds at most one chunk at the host's key bound (then that chunk is the split's only one), or
// there is one split per head (then the first two tiles sit at 16w and 16w + 16W) -- so their
// loads go out with the queries, in the shadow of the cursor / kv_len read (prefix mode only;
// FUSED only with Tq = 1, where the one new key is taken from k_new/v_new registers loaded
// alongside, where each tile is used). If the device length exceeds the bound so that a split
// holds more than one chunk, the early loads are dropped and the split is loaded again.
template <typename T, int D, typename OutT, bool FUSED, bool SPEC, int W>
__global__ void __launch_bounds__(DecShape<W>::threads) k_attn_decode(AttnArgs a, int group, float* ws,
                                                                        int n_splits) {
  constexpr int CH = DecShape<W>::chunk;
  constexpr int NT = DecShape<W>::threads;
  constexpr bool PATCH = FUSED && SPEC;
  // P V in fp16 (V converted while staged) for bf16 inputs with an fp32 output, where a
  // bf16-rounded P would be the dominant error of the result
  constexpr bool PV16 = std::is_same<T, bf16_t>::value && std::is_same<OutT, float>::value;
  typedef typename std::conditional<PV16, f16_t, T>::type TP;
  typedef DecMma<T> MQ;
  typedef DecMma<TP> MP;
  typedef typename MQ::vec8 vec8;
  typedef typename MP::vec4 pvec4;
  constexpr int DQ = D / 32;   // 32-wide d steps of S^T
  constexpr int CB = D / 16;   // 16-column output blocks
  constexpr int VU = D / 32;   // 16-byte V pieces per lane per tile
  // V tile row pitch: 32 bytes past a multiple of 256, so the 8 key rows one half-wavefront
  // reads in a transposed read fall on distinct banks
  constexpr int LDV = D == 128 ? D + 16 : D + 80;
  __shared__ __attribute__((aligned(16))) union {
    TP v[W][kDecTile * LDV];             // per-wavefront V tile
    float4 o[W][4][D];                   // after the tile loop: per-wavefront o, by row quad
    float wt[kDecMaxSplits][kDecRows];   // cross-split merge: weight of each partial
  } sm;
  __shared__ __attribute__((aligned(16))) float st_m[W][kDecRows];
  __shared__ __attribute__((aligned(16))) float st_l[W][kDecRows];
  __shared__ int last_s;

  // Every kernel argument in one batch of scalar loads and one wait: left to itself the
  // compiler loads each where it is first used, three dependent round trips before the cursor
  // can even be read. The asm takes them all as inputs and passes the split count through to
  // the workgroup mapping below, so it sits at the top; it is not volatile and touches no
  // memory, so the metadata reads after it stay scalar loads.
  asm("" : "+s"(n_splits) : "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.out), "s"(a.lse), "s"(a.kv_len_dev), "s"(a.cu),
      "s"(a.err), "s"(a.k_new), "s"(a.v_new), "s"(a.cursor), "s"(a.kv_len_out), "s"(ws));
  asm("" : "+s"(n_splits) : "s"(a.B), "s"(a.Tq), "s"(a.Hq), "s"(a.Hkv), "s"(a.cap), "s"(a.kv_len_host),
      "s"(a.mask), "s"(a.block), "s"(a.full_cap), "s"(a.scale), "s"(a.scale_log2), "s"(group));

  // Workgroup -> (split, b, g). Dispatch deals consecutive workgroup ids to the 8 XCDs in turn;
  // when B*Hkv is a multiple of 8, the ids are arranged so that every split of one (b, g)
  // lands on the same XCD: its partials meet in one L2, and from one step to the next the same
  // XCD reads the same rows of the head's K/V, which stay in its L2.
  const int BH = a.B * a.Hkv;
  int split, bg;
  if ((BH & 7) == 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int kq = k / n_splits;
    bg = x + 8 * kq;
    split = k - kq * n_splits;
  } else {
    bg = blockIdx.x / n_splits;
    split = blockIdx.x - bg * n_splits;
  }
  // (uniform values held in scalar registers: the metadata reads below then stay scalar loads)
  const int g = __builtin_amdgcn_readfirstlane(bg % a.Hkv), b = __builtin_amdgcn_readfirstlane(bg / a.Hkv);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n16 = lane & 15, G = lane >> 4;
  const int R = a.Tq * group;
  // workspace: arrival counters first (a fixed place for any split count), then partials
  int* counters = (int*)ws;
  float* ws_o = ws + dec_counter_floats(a.B, a.Hkv);
  float* ws_ml = ws_o + dec_o_floats(a.B, a.Hkv, D, n_splits);

  // query row n16 as the B operand of S^T (independent of the metadata: issued first).
  // Rows past R (padding up to the 16-row MFMA block) repeat row R-1: every row has its own
  // softmax and P V rows, so a repeated row changes no other row, and rows past R are never
  // written. No lane-divergent branch here: it would turn the uniform values computed around it
  // into vector registers (and the metadata reads that use them into vector loads), and zeroing
  // the padding would wait for the query loads before the tile loads go out.
  vec8 qb[DQ];
  {
    const int r = min(n16, R - 1);
    const int t = r / group, hh = r - t * group;
    const T* qp = (const T*)a.q + (((int64_t)b * a.Tq + t) * a.Hq + g * group + hh) * D + 8 * G;
#pragma unroll
    for (int c = 0; c < DQ; ++c) qb[c] = *(const vec8*)(qp + 32 * c);
  }

  // fused step: wave 0 of split 0 copies this head's slice of the new rows into the cache.
  // The sources do not depend on the cursor, so their loads go out here, before the cursor
  // read; the stores follow once this wave's tile loads are issued, so neither waits for the
  // copy. Lane (t, c8): row t, 16-byte granule c8 (Tq * D/8 <= 64 on this path).
  constexpr int VPR = D / 8;
  const int64_t rstride = (int64_t)a.Hkv * D;
  const bool copier = FUSED && split == 0 && wave == 0;  // wave-uniform
  const int cp_t = min(lane / VPR, a.Tq - 1), cp_c8 = lane % VPR;
  uint4 cpk, cpv;  // set and used only by the copier wave (not with early loads, see below)
  if (copier && !PATCH) {
    const int64_t src = ((int64_t)b * a.Tq + cp_t) * rstride + (int64_t)g * D + 8 * cp_c8;
    cpk = *(const uint4*)((const T*)a.k_new + src);
    cpv = *(const uint4*)((const T*)a.v_new + src);
  }

  // Tile loads. K: lane (G, n16) takes key tile + n16, d = 32c + 8G .. +8 (the A operand of
  // S^T). V: lane takes key tile + lane/4, d = 8(4u + lane%4) .. +8 (whole rows per 4 lanes).
  // Every load is issued unconditionally -- keys past the end read a row that exists (clamped)
  // and are zeroed where they are used -- so the outstanding loads form a fixed sequence and
  // the waits before each tile's math cover only that tile.
  constexpr int LT = DQ + VU;  // loads per tile
  auto load_rows = [&](const T* kb_, const T* vb_, const T* kn_, const T* vn_, int cur_, int jk,
                       int jv, uint4* kr, uint4* vr) {
    const T* kp = (FUSED && jk >= cur_) ? kn_ : kb_;
#pragma unroll
    for (int c = 0; c < DQ; ++c) kr[c] = *(const uint4*)(kp + (int64_t)jk * rstride + 32 * c + 8 * G);
    const T* vp = (FUSED && jv >= cur_) ? vn_ : vb_;
#pragma unroll
    for (int u = 0; u < VU; ++u) vr[u] = *(const uint4*)(vp + (int64_t)jv * rstride + 8 * (4 * u + (lane & 3)));
  };

  // SPEC: the new row in both lane layouts, then the first tile (and with one split the second)
  // of this wavefront, loaded before the length is known. Rows are clamped to the slab, so every
  // address is in bounds whatever the length.
  const int t0s = split * CH + kDecTile * wave;
  uint4 k0[DQ], v0[VU], k1[DQ], v1[VU];
  uint4 kn[DQ], vn[VU];  // PATCH only: the new row (Tq = 1) in the K and V lane layouts
  if constexpr (SPEC) {
    if constexpr (FUSED) {
      const int64_t nrow = (int64_t)b * rstride + (int64_t)g * D;  // Tq = 1: row b of k_new
#pragma unroll
      for (int c = 0; c < DQ; ++c) kn[c] = *(const uint4*)((const T*)a.k_new + nrow + 32 * c + 8 * G);
#pragma unroll
      for (int u = 0; u < VU; ++u) vn[u] = *(const uint4*)((const T*)a.v_new + nrow + 8 * (4 * u + (lane & 3)));
    }
    const T* kb0 = (const T*)a.k + (int64_t)b * a.cap * rstride + (int64_t)g * D;
    const T* vb0 = (const T*)a.v + (int64_t)b * a.cap * rstride + (int64_t)g * D;
    load_rows(kb0, vb0, nullptr, nullptr, 0x7fffffff, min(t0s + n16, a.cap - 1),
              min(t0s + (lane >> 2), a.cap - 1), k0, v0);
    if (n_splits == 1)
      load_rows(kb0, vb0, nullptr, nullptr, 0x7fffffff, min(t0s + CH + n16, a.cap - 1),
                min(t0s + CH + (lane >> 2), a.cap - 1), k1, v1);
  }

  // The copier's stores. With early loads the row is in kn (lane (G, n16) holds granules 4c + G,
  // c < DQ: lanes 0, 16, 32, 48 cover the row) and vn (lane l < 4 holds granules 4u + l).
  auto copy_new_rows = [&](int cur_, const KeySet& ks_) {
    if (!copier || !ks_.ok) return;
    if constexpr (PATCH) {
      T* kd = (T*)a.k + (ks_.base_row + cur_) * rstride + (int64_t)g * D;
      T* vd = (T*)a.v + (ks_.base_row + cur_) * rstride + (int64_t)g * D;
      if (n16 == 0) {
#pragma unroll
        for (int c = 0; c < DQ; ++c) *(uint4*)(kd + 32 * c + 8 * G) = kn[c];
      }
      if (lane < 4) {
#pragma unroll
        for (int u = 0; u < VU; ++u) *(uint4*)(vd + 8 * (4 * u + lane)) = vn[u];
      }
    } else if (lane < a.Tq * VPR) {
      const int64_t dst = (ks_.base_row + cur_ + cp_t) * rstride + (int64_t)g * D + 8 * cp_c8;
      *(uint4*)((T*)a.k + dst) = cpk;
      *(uint4*)((T*)a.v + dst) = cpv;
    }
  };

  // the key range: a rejected batch element (or a full cache) is one split with no keys
  int cur = 0;  // fused step: the write position of this step
  KeySet ks;
  if constexpr (FUSED) {
    cur = *a.cursor;
    const bool fits = cur >= 0 && (int64_t)cur + a.Tq <= a.cap;
    ks.base_row = (int64_t)b * a.cap;
    ks.len = fits ? cur + a.Tq : 0;
    ks.visit = ks.len;
    ks.ok = fits;
    if (!fits && threadIdx.x == 0 && split == 0 && g == 0 && b == 0) report(a.err, SKV_DEV_CURSOR_FULL);
  } else {
    ks = key_set(a, b);
    if (!ks.ok && threadIdx.x == 0 && split == 0 && g == 0) report(a.err, dev_error_bit(a));
  }
  // this split's share of the visited rows, in whole chunks; splits at or past n_active hold no
  // keys
  int per = (ks.visit + n_splits - 1) / n_splits;
  per = (per + CH - 1) / CH * CH;
  const int n_active = ks.ok ? (ks.visit + per - 1) / per : 1;
  const int start = split * per;
  const int end = ks.ok ? min(ks.visit, start + per) : 0;

  // fused step: every workgroup has read the cursor once it counts itself in here; the count
  // comes back while the workgroup works and is looked at when it leaves
  int reader_rank = 0;
  auto count_reader = [&]() {
    if constexpr (FUSED) {
      if (threadIdx.x == 0)
        reader_rank = __hip_atomic_fetch_add(&counters[BH], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto advance_cursor_if_last_reader = [&]() {
    if constexpr (FUSED) {
      if (threadIdx.x == 0 && reader_rank == (int)gridDim.x - 1) {
        if (ks.ok) {
          if (a.kv_len_out)
            for (int bb = 0; bb < a.B; ++bb) a.kv_len_out[bb] = cur + a.Tq;
          *a.cursor = cur + a.Tq;
        }
        __hip_atomic_store(&counters[BH], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  if (split >= n_active) {
    count_reader();
    advance_cursor_if_last_reader();
    return;
  }

  // last visible key of row n16 within this split (padding rows see the whole split)
  int lim = end - 1;
  if (n16 < R) {
    const int rl = row_limit(a.mask, a.block, ks.len - a.Tq + n16 / group, ks.len);
    lim = rl < lim ? rl : lim;
  }

  const T* kbase = (const T*)a.k + ks.base_row * rstride + (int64_t)g * D;
  const T* vbase = (const T*)a.v + ks.base_row * rstride + (int64_t)g * D;
  // fused step: key j >= cur is new row j - cur of k_new/v_new (rows of batch element b)
  const T* knew = nullptr;
  const T* vnew = nullptr;
  if constexpr (FUSED) {
    knew = (const T*)a.k_new + (int64_t)b * a.Tq * rstride + (int64_t)g * D - (int64_t)cur * rstride;
    vnew = (const T*)a.v_new + (int64_t)b * a.Tq * rstride + (int64_t)g * D - (int64_t)cur * rstride;
  }
  auto load_tile = [&](int tile, uint4* kr, uint4* vr) {
    load_rows(kbase, vbase, knew, vnew, cur, min(tile + n16, max(end - 1, 0)),
              min(tile + (lane >> 2), max(end - 1, 0)), kr, vr);
  };
  // Keys at or past `end` count as zero rows. The mask is applied where the tile is used and
  // passes through an empty asm: with a visible condition the compiler would turn the
  // zeroing back into a load under that condition.
  auto keep_mask = [&](int key) {
    unsigned k = key < end ? ~0u : 0u;
    asm volatile("" : "+v"(k));
    return k;
  };
  auto masked = [](uint4 x, unsigned k) { return make_uint4(x.x & k, x.y & k, x.z & k, x.w & k); };
  // PATCH: in an early-loaded tile, key cur (the new row) comes from the k_new/v_new registers
  // (the tile was read from the cache before this step's row is written). Tiles loaded after the
  // cursor was read take it from k_new/v_new already.
  auto pick = [](uint4 x, uint4 y, bool use_y) {
    return make_uint4(use_y ? y.x : x.x, use_y ? y.y : x.y, use_y ? y.z : x.z, use_y ? y.w : x.w);
  };
  auto patch_tile = [&](int tile, uint4* kr, uint4* vr) {
    if constexpr (PATCH) {
      const bool new_k = tile + n16 == cur, new_v = tile + (lane >> 2) == cur;
#pragma unroll
      for (int c = 0; c < DQ; ++c) kr[c] = pick(kr[c], kn[c], new_k);
#pragma unroll
      for (int u = 0; u < VU; ++u) vr[u] = pick(vr[u], vn[u], new_v);
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{};
  const float c2 = a.scale_log2;
  TP* vt = sm.v[wave];

  // One tile's math: S^T, online softmax, P V.
  auto process = [&](int tile, const uint4* kraw, const uint4* vraw) {
    const unsigned kk = keep_mask(tile + n16), vk = keep_mask(tile + (lane >> 2));
    // V tile to LDS (row = key, converted to the P V type)
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      TP* dst = vt + (lane >> 2) * LDV + 8 * (4 * u + (lane & 3));
      const uint4 vm = masked(vraw[u], vk);
      if constexpr (PV16) {
        const bf16_t* e = (const bf16_t*)&vm;
        typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 h8;
        h8 hv;
#pragma unroll
        for (int k = 0; k < 8; ++k) hv[k] = (f16_t)(float)e[k];
        *(h8*)dst = hv;
      } else {
        *(uint4*)dst = vm;
      }
    }

    // S^T = K Q^T: s[j] = score(key tile + 4G + j, row n16)
    f32x4 s = f32x4{};
#pragma unroll
    for (int c = 0; c < DQ; ++c)
      s = MQ::qk(__builtin_bit_cast(vec8, masked(kraw[c], kk)), qb[c], s);
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = tile + 4 * G + j <= lim ? s[j] : -INFINITY;
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = max_xor32(max_xor16(mt));
    const bool grow = (mt - m) * c2 > kDecRescaleLog2;  // NaN (no move) when both are -inf
    const float m_new = grow ? mt : m;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c2);
    const float mc = m_use * c2;
    const pvec4 pa = MP::pack(__builtin_amdgcn_exp2f(fmaf(sv[0], c2, -mc)),
                              __builtin_amdgcn_exp2f(fmaf(sv[1], c2, -mc)),
                              __builtin_amdgcn_exp2f(fmaf(sv[2], c2, -mc)),
                              __builtin_amdgcn_exp2f(fmaf(sv[3], c2, -mc)));
    lsum = MP::sum4(pa, lsum * alpha);
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // O rows 4G + j take the factor of row 4G + j, held by lane 4G + j
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * G + j, 64);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[cb][j] *= al[j];
    }

    // P V: B operand V[key 4G + t][16cb + n16], t = 0..3, by one transposed read: lane k of
    // each 16-lane group points at V[4G + k/4][16cb + 4(k%4)]
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const TP* vp = vt + (4 * G + (n16 >> 2)) * LDV + 16 * cb + 4 * (n16 & 3);
      const dec_s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_s16x4*)vp);
      o[cb] = MP::pv(pa, __builtin_bit_cast(pvec4, x), o[cb]);
    }
    // the V tile is rewritten by this wavefront's next tile
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // This wavefront's tiles are t0, t0 + CH, ... below end (wave-uniform).
  const int t0 = start + kDecTile * wave;
  const int n_tiles = end > t0 ? (end - t0 + CH - 1) / CH : 0;
  if (SPEC && per == CH) {
    // the early tile is this wavefront's only one (t0 == t0s)
    if constexpr (FUSED) {
      copy_new_rows(cur, ks);
      count_reader();
    }
    if (n_tiles > 0) {
      patch_tile(t0, k0, v0);
      process(t0, k0, v0);
    }
  } else if (n_tiles > 0) {  // then end >= 1 and every clamped row lies in the visited range
    // Two tiles ahead: three register buffers in a loop unrolled by three, so no buffer is
    // copied into another (a copy would wait for the newest loads), and the 0-2 remaining
    // tiles after the loop. Before the loop one wait retires everything issued ahead of the
    // first two tiles' loads (the queries, the new rows' source loads), so the waits the
    // compiler places in the loop count only tile loads; the copier's stores follow it. With
    // one split per head the first two tiles were loaded early (t0 == t0s).
    uint4 k2[DQ], v2[VU];
    if (!(SPEC && n_splits == 1)) {
      load_tile(t0, k0, v0);
      load_tile(t0 + CH, k1, v1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcntTwoTiles<LT>());
    if constexpr (FUSED) {
      copy_new_rows(cur, ks);
      count_reader();
    }
    if (SPEC && n_splits == 1) {
      patch_tile(t0, k0, v0);
      patch_tile(t0 + CH, k1, v1);
    }
    int i = 0;
    for (; i + 3 <= n_tiles; i += 3) {
      const int tile = t0 + i * CH;
      load_tile(tile + 2 * CH, k2, v2);
      process(tile, k0, v0);
      load_tile(tile + 3 * CH, k0, v0);
      process(tile + CH, k1, v1);
      load_tile(tile + 4 * CH, k1, v1);
      process(tile + 2 * CH, k2, v2);
    }
    if (i < n_tiles) process(t0 + i * CH, k0, v0);
    if (i + 1 < n_tiles) process(t0 + (i + 1) * CH, k1, v1);
  } else if constexpr (FUSED) {
    copy_new_rows(cur, ks);  // (the copier wave always has tiles when the step is valid)
    count_reader();
  }

  // row n16's sum: the four lane groups hold different keys of it
  lsum = sum_xor32(sum_xor16(lsum));
  const int RQ = (R + 3) >> 2;  // row quads in use
  __syncthreads();  // every wavefront is done with its V tile: the union becomes the output stage
  if (G == 0) {
    st_m[wave][n16] = m;
    st_l[wave][n16] = lsum;
  }
  if (G < RQ) {  // lane (G, n16) holds rows 4G .. 4G+3 of columns 16cb + n16
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sm.o[wave][G][16 * cb + n16] = make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
  }
  __syncthreads();

  // merge the wavefronts: thread -> (row quad, column)
  const __amdgpu_buffer_rsrc_t ro = ws_rsrc(ws_o, dec_o_floats(a.B, a.Hkv, D, n_splits));
  const __amdgpu_buffer_rsrc_t rml = ws_rsrc(ws_ml, dec_ml_floats(a.B, a.Hkv, n_splits));
  for (int p = threadIdx.x; p < RQ * D; p += NT) {
    const int rq = p / D, col = p - rq * D;
    float4 mw[W], lw[W], ow[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      mw[w] = *(const float4*)&st_m[w][4 * rq];
      lw[w] = *(const float4*)&st_l[w][4 * rq];
      ow[w] = sm.o[w][rq][col];
    }
    float Mj[4], Lj[4], Oj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, f4_get(mw[w], j));
      const float mu = M == -INFINITY ? 0.f : M;
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float e = __builtin_amdgcn_exp2f((f4_get(mw[w], j) - mu) * c2);
        L = fmaf(e, f4_get(lw[w], j), L);
        O = fmaf(e, f4_get(ow[w], j), O);
      }
      Mj[j] = M;
      Lj[j] = L;
      Oj[j] = O;
    }
    if (n_active == 1) {  // the workgroup saw every key: its merge is the output
      float4 v;
      v.x = Lj[0] > 0.f ? Oj[0] / Lj[0] : 0.f;  // L = 0: the batch element was rejected
      v.y = Lj[1] > 0.f ? Oj[1] / Lj[1] : 0.f;
      v.z = Lj[2] > 0.f ? Oj[2] / Lj[2] : 0.f;
      v.w = Lj[3] > 0.f ? Oj[3] / Lj[3] : 0.f;
      write_quad<OutT>(a, D, group, b, g, rq, col, v);
      if (a.lse && col == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * rq + j < R) write_lse(a, group, b, g, 4 * rq + j, Mj[j], Lj[j]);
    } else {
      store_coherent(ro, (dec_o_quad(b, g, split, rq, a.Hkv, n_splits, D) + col) * 4,
                     make_float4(Oj[0], Oj[1], Oj[2], Oj[3]));
      if (col == 0) {
        const size_t base = dec_ml_base(b, g, split, a.Hkv, n_splits);
        store_coherent(rml, base + 4 * rq, make_float4(Mj[0], Mj[1], Mj[2], Mj[3]));
        store_coherent(rml, base + kDecRows + 4 * rq, make_float4(Lj[0], Lj[1], Lj[2], Lj[3]));
      }
    }
  }

  if (n_active > 1) {
    // every store of the workgroup has completed before its arrival is counted
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
      int* cnt = &counters[b * a.Hkv + g];
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == n_active - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_s = last;
    }
    __syncthreads();
    if (last_s) {
      // The partials are read with sc1 loads, the form agent-scope atomic loads take: they see
      // every store that completed before its workgroup was counted, with no cache invalidate.
      // The fence keeps the compiler from moving them above the arrival count.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      merge_splits<D, OutT, NT>(a, group, RQ, ws_o + dec_o_quad(b, g, 0, 0, a.Hkv, n_splits, D) * 4, rml,
                                sm.wt, b, g, n_active, n_splits);
    }
  }
  advance_cursor_if_last_reader();
}

// Split count used by both the launcher and the workspace query. Splits are whole chunks
// (64 keys: one 16-key tile per wavefront), at most one workgroup per CU over the chip and at
// most 32 per head. When the key bound fits in that many single-chunk splits, each split holds
// one chunk, so every wavefront's tile is known before the length is read; longer bounds take
// about 128 keys per split (fewer, longer splits measured faster from 4K to 32K keys, where
// the merge of many partials cost more than the extra parallelism gave).
int decode_splits(int B, int Hkv, int max_len) {
  constexpr int CH = DecShape<kDecWaves>::chunk;
  int target = 256 / (B * Hkv);
  if (target < 1) target = 1;
  if (target > kDecMaxSplits) target = kDecMaxSplits;
  const int one_chunk = (max_len + CH - 1) / CH;
  if (one_chunk <= target) return one_chunk < 1 ? 1 : one_chunk;
  const int by_len = (max_len + 2 * CH - 1) / (2 * CH);
  const int s = by_len < target ? by_len : target;
  return s < 1 ? 1 : s;
}

size_t decode_workspace_bytes(int B, int Hkv, int D, int n_splits) {
  return (dec_counter_floats(B, Hkv) + dec_o_floats(B, Hkv, D, n_splits) +
          dec_ml_floats(B, Hkv, n_splits)) * sizeof(float);
}

template <typename T, int D, typename OutT, bool FUSED, int W>
static hipError_t launch_decode_w(const AttnArgs& a, int group, float* ws, int n_splits,
                                  int key_bound, hipStream_t s) {
  const int64_t blocks = (int64_t)n_splits * a.B * a.Hkv;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(DecShape<W>::threads);
  // early tile loads: prefix mode, one new row per fused step, and the first tiles' places
  // fixed by the launch (one chunk per split at the bound, or one split)
  const bool spec = a.cu == nullptr && (!FUSED || a.Tq == 1) &&
                    (n_splits == 1 || (int64_t)n_splits * DecShape<W>::chunk >= key_bound);
  if (spec)
    hipLaunchKernelGGL((k_attn_decode<T, D, OutT, FUSED, true, W>), grid, block, 0, s, a, group, ws, n_splits);
  else
    hipLaunchKernelGGL((k_attn_decode<T, D, OutT, FUSED, false, W>), grid, block, 0, s, a, group, ws, n_splits);
  return hipGetLastError();
}

template <typename T, int D, typename OutT, bool FUSED>
static hipError_t launch_decode_f(const AttnArgs& a, int group, float* ws, int n_splits,
                                  int key_bound, hipStream_t s) {
  return launch_decode_w<T, D, OutT, FUSED, kDecWaves>(a, group, ws, n_splits, key_bound, s);
}

template <typename T, int D, typename OutT>
static hipError_t launch_decode_t(const AttnArgs& a, int group, float* ws, int n_splits,
                                  int key_bound, hipStream_t s) {
  return a.cursor ? launch_decode_f<T, D, OutT, true>(a, group, ws, n_splits, key_bound, s)
                  : launch_decode_f<T, D, OutT, false>(a, group, ws, n_splits, key_bound, s);
}

hipError_t launch_attn_decode(const AttnArgs& a, int dtype, int out_dtype, int D, void* ws,
                              int n_splits, int key_bound, hipStream_t s) {
  const int group = a.Hq / a.Hkv;
  float* w = (float*)ws;
  if (dtype == SKV_BF16) {
    if (D == 128)
      return out_dtype == SKV_F32 ? launch_decode_t<bf16_t, 128, float>(a, group, w, n_splits, key_bound, s)
                                  : launch_decode_t<bf16_t, 128, bf16_t>(a, group, w, n_splits, key_bound, s);
    return out_dtype == SKV_F32 ? launch_decode_t<bf16_t, 64, float>(a, group, w, n_splits, key_bound, s)
                                : launch_decode_t<bf16_t, 64, bf16_t>(a, group, w, n_splits, key_bound, s);
  }
  if (D == 128)
    return out_dtype == SKV_F32 ? launch_decode_t<f16_t, 128, float>(a, group, w, n_splits, key_bound, s)
                                : launch_decode_t<f16_t, 128, f16_t>(a, group, w, n_splits, key_bound, s);
  return out_dtype == SKV_F32 ? launch_decode_t<f16_t, 64, float>(a, group, w, n_splits, key_bound, s)
                              : launch_decode_t<f16_t, 64, f16_t>(a, group, w, n_splits, key_bound, s);
}

}  // namespace skv
