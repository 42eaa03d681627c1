// Decode-sized attention (Tq <= 4): split-K over the key range, then an LSE-weighted merge.
//
// Each decode step i attends its single new query to the active prefix kv_len = T + i + 1
// (fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA",
// section Change); the step reads 2*kv_len*Hkv*D*elem bytes of K/V and does almost no math
// per byte, so the kernel is built to stream K/V at HBM rate:
//   * one wavefront per (split, KV head, batch element); the key range [0, visit) is cut into
//     gridDim.x equal parts computed on the device from kv_len, so a fixed grid (graph replay
//     with a device kv_len) still spreads any length over every wavefront;
//   * all query rows of a GQA group (Hq/Hkv heads x Tq rows, <= 16) share each K/V load:
//     S = Q K^T on v_mfma_f32_16x16x32 (K straight from global memory in the B-operand
//     layout, the group's query rows as A), softmax in fp32, and P V on the vector ALUs with
//     P kept in fp32 (each lane owns 8 output columns of a quarter of the keys);
//   * every split writes its unnormalised (m, l, o) to the caller's workspace; the last split
//     of each (b, KV head) to finish merges them with weights exp(m_s - max m), so one launch
//     is the whole step (the workspace's arrival counters start at zero and are left at zero).
#include "common.h"

namespace skv {

template <typename T> struct Mfma16;
template <> struct Mfma16<bf16_t> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<f16_t> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kDecBN = 64;   // keys per tile
constexpr int kDecRows = 16; // row slots per (b, KV head) in the workspace

__host__ __device__ __forceinline__ size_t dec_counter_floats(int B, int Hkv) {
  return (((size_t)B * Hkv + 1 + 63) / 64) * 64;  // B*Hkv split counters + 1, 256-byte multiple
}
__host__ __device__ __forceinline__ size_t dec_o_floats(int B, int Hkv, int D, int n_splits) {
  return (size_t)B * Hkv * kDecRows * n_splits * D;
}
__host__ __device__ __forceinline__ size_t dec_ml_floats(int B, int Hkv, int n_splits) {
  return ((size_t)B * Hkv * kDecRows * n_splits * 2 + 3) & ~(size_t)3;  // keep 16-byte alignment
}

__device__ __forceinline__ size_t dec_part_index(int b, int g, int r, int split, int Hkv,
                                                 int n_splits) {
  return (((size_t)b * Hkv + g) * kDecRows + r) * n_splits + split;
}

template <typename T>
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  const T* e = (const T*)&u;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = to_f32(e[i]);
}

// Merge the n_splits partials of the R rows of (b, g) and write the output rows. Lane layout:
// row r0 + lane/16 of each pass of 4 rows, columns [8*(lane%16), +8). One online pass over the
// splits (running max M, weights exp2((m_s - M) * scale * log2 e)); the loads of 8 splits are
// issued together and nothing in the loop branches on loaded data.
template <int D, typename OutT>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int group, const float* ws_o,
                                           const float* ws_ml, int b, int g, int R, int n_splits,
                                           int lane) {
  constexpr int kBatch = 8;
  const int dc = lane & 15;
  const bool col_ok = dc < D / 8;
  const float c2 = a.scale_log2;
  for (int r0 = 0; r0 < R; r0 += 4) {
    const int r = r0 + (lane >> 4);
    const bool row_ok = r < R;
    const size_t p0 = dec_part_index(b, g, row_ok ? r : 0, 0, a.Hkv, n_splits);
    float M = -INFINITY, L = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
      float2 ml[kBatch];
      float4 oa[kBatch], ob[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int sp = s0 + u;
        const bool ok = sp < n_splits;
        ml[u] = ok ? *(const float2*)(ws_ml + 2 * (p0 + sp)) : make_float2(-INFINITY, 0.f);
        const float* po = ws_o + (p0 + (ok ? sp : 0)) * D + 8 * dc;
        oa[u] = (ok && col_ok) ? *(const float4*)po : make_float4(0.f, 0.f, 0.f, 0.f);
        ob[u] = (ok && col_ok) ? *(const float4*)(po + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float m_new = fmaxf(M, ml[u].x);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float wa = __builtin_amdgcn_exp2f((M - m_use) * c2);       // rescale of the sum so far
        const float wb = __builtin_amdgcn_exp2f((ml[u].x - m_use) * c2); // weight of split s
        L = L * wa + ml[u].y * wb;
        o[0] = o[0] * wa + oa[u].x * wb;
        o[1] = o[1] * wa + oa[u].y * wb;
        o[2] = o[2] * wa + oa[u].z * wb;
        o[3] = o[3] * wa + oa[u].w * wb;
        o[4] = o[4] * wa + ob[u].x * wb;
        o[5] = o[5] * wa + ob[u].y * wb;
        o[6] = o[6] * wa + ob[u].z * wb;
        o[7] = o[7] * wa + ob[u].w * wb;
        M = m_new;
      }
    }
    if (!row_ok) continue;
    const int t = r / group, h = g * group + (r - t * group);
    OutT* out = (OutT*)a.out + (((int64_t)b * a.Tq + t) * a.Hq + h) * D + 8 * dc;
    const float inv = L > 0.f ? 1.f / L : 0.f;  // L = 0: the batch element was rejected
    if (col_ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = from_f32<OutT>(o[e] * inv);
    }
    if (a.lse && dc == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.Tq + t] = L > 0.f ? M * a.scale + logf(L) : -INFINITY;
  }
}

// NR: query rows per KV head rounded up to 4, 8 or 16 (R = Tq * Hq/Hkv <= NR).
// One launch does the whole decode attention: every wavefront writes its split's partials,
// and the last wavefront of each (b, KV head) to arrive -- counted with a device-scope
// atomic in the workspace -- merges them and resets the counter to zero for the next call.
// FUSED: one launch per decode step with the write cursor on the device (attn_decode_step):
// c = *cursor; the new rows k_new/v_new [B, Tq, Hkv, D] are written to cache rows c .. c+Tq-1
// and attended over as keys c .. c+Tq-1 straight from the sources (no wavefront of this launch
// reads a cache row another one writes); the last (b, g) merge to finish sets *cursor = c+Tq
// and kv_len_out[:] = c+Tq, after every wavefront has read the cursor.
template <typename T, int D, int NR, typename OutT, bool FUSED>
__global__ void __launch_bounds__(64) k_attn_decode(AttnArgs a, int group, float* ws,
                                                    int n_splits) {
  typedef typename Mfma16<T>::vec vec;
  constexpr int DQ = D / 32;  // 32-wide d chunks of the QK^T contraction
  __shared__ __attribute__((aligned(16))) float P[kDecBN][kDecRows];
  __shared__ float alpha_s[kDecRows];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 15, quad = lane >> 4;
  const int R = a.Tq * group;
  // workspace: arrival counters first (a fixed place for any split count), then partials
  int* counters = (int*)ws;
  float* ws_o = ws + dec_counter_floats(a.B, a.Hkv);
  float* ws_ml = ws_o + dec_o_floats(a.B, a.Hkv, D, n_splits);

  // a rejected batch element still takes part in the arrival count, with empty splits
  int cur = 0;  // fused step: the write position of this step
  KeySet ks;
  if constexpr (FUSED) {
    cur = *a.cursor;
    const bool fits = cur >= 0 && (int64_t)cur + a.Tq <= a.cap;
    ks.base_row = (int64_t)b * a.cap;
    ks.len = fits ? cur + a.Tq : 0;
    ks.visit = ks.len;
    ks.ok = fits;
    if (!fits && lane == 0 && split == 0 && g == 0 && b == 0) report(a.err, SKV_DEV_CURSOR_FULL);
  } else {
    ks = key_set(a, b);
    if (!ks.ok && lane == 0 && split == 0 && g == 0) report(a.err, dev_error_bit(a));
  }
  // this split's share of the visited rows, in whole 16-key steps
  int per = (ks.visit + n_splits - 1) / n_splits;
  per = (per + 15) & ~15;
  const int start = split * per;
  const int end = ks.ok ? min(ks.visit, start + per) : 0;

  // A operand: query row `col` (row r = t*group + hh -> head g*group + hh, query t)
  vec qa[DQ];
  {
    const int r = col;
    if (r < R) {  // independent of kv_len, so these loads overlap the metadata load
      const int t = r / group, hh = r - t * group;
      const T* qp = (const T*)a.q + (((int64_t)b * a.Tq + t) * a.Hq + g * group + hh) * D + 8 * quad;
#pragma unroll
      for (int c = 0; c < DQ; ++c) qa[c] = *(const vec*)(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < DQ; ++c) qa[c] = vec{};
    }
  }
  // accumulator rows held by this lane in the S phase: r = 4*quad + j
  int pos[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * quad + j;
    pos[j] = ks.len - a.Tq + (r < R ? r / group : 0);
  }
  // last visible key of each row within this split: one compare per score, no branches
  int lim[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rl = row_limit(a.mask, a.block, pos[j], ks.len);
    lim[j] = rl < end - 1 ? rl : end - 1;
  }
  float m[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
  }
  float acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  const int64_t rstride = (int64_t)a.Hkv * D;
  const T* kbase = (const T*)a.k + ks.base_row * rstride + (int64_t)g * D;
  const T* vbase = (const T*)a.v + ks.base_row * rstride + (int64_t)g * D;
  // fused step: key j >= cur is new row j - cur of k_new/v_new (rows of batch element b)
  const T* knew = nullptr;
  const T* vnew = nullptr;
  if constexpr (FUSED) {
    knew = (const T*)a.k_new + (int64_t)b * a.Tq * rstride + (int64_t)g * D - (int64_t)cur * rstride;
    vnew = (const T*)a.v_new + (int64_t)b * a.Tq * rstride + (int64_t)g * D - (int64_t)cur * rstride;
    if (split == 0 && ks.ok) {  // this head's slice of the new rows goes into the cache
      constexpr int VPR = D / 8;
      for (int i = lane; i < a.Tq * VPR; i += 64) {
        const int t = i / VPR, c8 = i - t * VPR;
        const int64_t row = cur + t;
        *(uint4*)((T*)a.k + ks.base_row * rstride + row * rstride + (int64_t)g * D + 8 * c8) =
            *(const uint4*)(knew + row * rstride + 8 * c8);
        *(uint4*)((T*)a.v + ks.base_row * rstride + row * rstride + (int64_t)g * D + 8 * c8) =
            *(const uint4*)(vnew + row * rstride + 8 * c8);
      }
    }
  }
  const float c2 = a.scale_log2;
  const int dc = col;    // PV phase: this lane's 8 output columns [8dc, 8dc+8)
  const int kg = quad;   // PV phase: keys kg, kg+4, ..., kg+60 of the tile
  const bool dc_ok = dc < D / 8;  // D = 64 leaves half of the lanes without columns

  for (int tile = start; tile < end; tile += kDecBN) {
    // issue every K and V load of the tile first
    uint4 kraw[4][DQ];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int j = tile + 16 * kb + col;
      const T* kb_ptr = (FUSED && j >= cur) ? knew : kbase;
#pragma unroll
      for (int c = 0; c < DQ; ++c)
        kraw[kb][c] = j < end ? *(const uint4*)(kb_ptr + (int64_t)j * rstride + 32 * c + 8 * quad)
                              : make_uint4(0, 0, 0, 0);
    }
    uint4 vraw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = tile + kg + 4 * i;
      const T* vb_ptr = (FUSED && j >= cur) ? vnew : vbase;
      vraw[i] = (j < end && dc_ok) ? *(const uint4*)(vb_ptr + (int64_t)j * rstride + 8 * dc)
                                   : make_uint4(0, 0, 0, 0);
    }
    // S = Q K^T: s[kb][j] = score(row 4*quad+j, key tile+16kb+col)
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int c = 0; c < DQ; ++c) {
        vec kv;
        __builtin_memcpy(&kv, &kraw[kb][c], sizeof(vec));
        s[kb] = Mfma16<T>::mma(qa[c], kv, s[kb]);
      }
    }
    float alpha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = tile + 16 * kb + col;
        const float sv = key <= lim[j] ? s[kb][j] : -INFINITY;
        s[kb][j] = sv;
        mt = fmaxf(mt, sv);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
      const float m_new = fmaxf(m[j], mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[j] = __builtin_amdgcn_exp2f((m[j] - m_use) * c2);
      const float mc = m_use * c2;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][j], c2, -mc));
        s[kb][j] = p;
        ps += p;
      }
      l[j] = l[j] * alpha[j] + ps;
      m[j] = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      *(float4*)&P[16 * kb + col][4 * quad] = make_float4(s[kb][0], s[kb][1], s[kb][2], s[kb][3]);
    if (col == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) alpha_s[4 * quad + j] = alpha[j];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float al = alpha_s[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v[8];
      unpack8<T>(vraw[i], v);
      const float* pr = P[kg + 4 * i];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float p = pr[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, v[e], acc[r][e]);
      }
    }
    __syncthreads();  // P and alpha_s are rewritten by the next tile
  }

  // row sums: each of the 16 lanes of a quad holds part of rows 4*quad+j
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l[j] += __shfl_xor(l[j], o, 64);
  // outputs: the four key groups (lane bits 4-5) hold partial sums of the same columns
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[r][e] += __shfl_xor(acc[r][e], 16, 64);
      acc[r][e] += __shfl_xor(acc[r][e], 32, 64);
    }
  if (kg == 0 && dc_ok) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r < R) {
        float* po = ws_o + dec_part_index(b, g, r, split, a.Hkv, n_splits) * D + 8 * dc;
        *(float4*)po = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
        *(float4*)(po + 4) = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
      }
    }
  }
  if (col == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * quad + j;
      if (r < R) {
        const size_t pi = dec_part_index(b, g, r, split, a.Hkv, n_splits);
        ws_ml[2 * pi] = m[j];
        ws_ml[2 * pi + 1] = l[j];
      }
    }
  }

  // arrive; the last split of this (b, g) merges. Writers only release their partials
  // (write-back); only the merging wavefront acquires (invalidate), so the L2 copy of the
  // cache that other wavefronts are still reading is not dropped by every arrival.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  int last = 0;
  if (lane == 0) {
    const int old = __hip_atomic_fetch_add(&counters[b * a.Hkv + g], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    last = old == n_splits - 1;
  }
  last = __shfl(last, 0, 64);
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  merge_rows<D, OutT>(a, group, ws_o, ws_ml, b, g, R, n_splits, lane);
  if (lane == 0)
    __hip_atomic_store(&counters[b * a.Hkv + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (FUSED) {
    // every wavefront of the launch read the cursor before it arrived: the last (b, g) merge
    // may move it
    int done = 0;
    if (lane == 0) {
      const int old = __hip_atomic_fetch_add(&counters[a.B * a.Hkv], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      done = old == a.B * a.Hkv - 1;
    }
    done = __shfl(done, 0, 64);
    if (!done) return;
    if (ks.ok) {
      if (a.kv_len_out)
        for (int bb = lane; bb < a.B; bb += 64) a.kv_len_out[bb] = cur + a.Tq;
      if (lane == 0) *a.cursor = cur + a.Tq;
    }
    if (lane == 0)
      __hip_atomic_store(&counters[a.B * a.Hkv], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Split count used by both the launcher and the workspace query.
int decode_splits(int B, int Hkv, int max_len) {
  const int tiles = (max_len + kDecBN - 1) / kDecBN;
  int target = 2048 / (B * Hkv);  // about two wavefronts per SIMD over the whole chip
  if (target < 1) target = 1;
  int s = tiles < target ? tiles : target;
  return s < 1 ? 1 : s;
}

size_t decode_workspace_bytes(int B, int Hkv, int D, int n_splits) {
  return (dec_counter_floats(B, Hkv) + dec_o_floats(B, Hkv, D, n_splits) +
          dec_ml_floats(B, Hkv, n_splits)) * sizeof(float);
}

template <typename T, int D, typename OutT, bool FUSED>
static hipError_t launch_decode_f(const AttnArgs& a, int group, float* ws, int n_splits,
                                  hipStream_t s) {
  const int R = a.Tq * group;
  dim3 grid(n_splits, a.Hkv, a.B), block(64);
  if (R <= 4)
    hipLaunchKernelGGL((k_attn_decode<T, D, 4, OutT, FUSED>), grid, block, 0, s, a, group, ws, n_splits);
  else if (R <= 8)
    hipLaunchKernelGGL((k_attn_decode<T, D, 8, OutT, FUSED>), grid, block, 0, s, a, group, ws, n_splits);
  else
    hipLaunchKernelGGL((k_attn_decode<T, D, 16, OutT, FUSED>), grid, block, 0, s, a, group, ws, n_splits);
  return hipGetLastError();
}

template <typename T, int D, typename OutT>
static hipError_t launch_decode_t(const AttnArgs& a, int group, float* ws, int n_splits,
                                  hipStream_t s) {
  return a.cursor ? launch_decode_f<T, D, OutT, true>(a, group, ws, n_splits, s)
                  : launch_decode_f<T, D, OutT, false>(a, group, ws, n_splits, s);
}

hipError_t launch_attn_decode(const AttnArgs& a, int dtype, int out_dtype, int D, void* ws,
                              int n_splits, hipStream_t s) {
  const int group = a.Hq / a.Hkv;
  float* w = (float*)ws;
  if (dtype == SKV_BF16) {
    if (D == 128)
      return out_dtype == SKV_F32 ? launch_decode_t<bf16_t, 128, float>(a, group, w, n_splits, s)
                                  : launch_decode_t<bf16_t, 128, bf16_t>(a, group, w, n_splits, s);
    return out_dtype == SKV_F32 ? launch_decode_t<bf16_t, 64, float>(a, group, w, n_splits, s)
                                : launch_decode_t<bf16_t, 64, bf16_t>(a, group, w, n_splits, s);
  }
  if (D == 128)
    return out_dtype == SKV_F32 ? launch_decode_t<f16_t, 128, float>(a, group, w, n_splits, s)
                                : launch_decode_t<f16_t, 128, f16_t>(a, group, w, n_splits, s);
  return out_dtype == SKV_F32 ? launch_decode_t<f16_t, 64, float>(a, group, w, n_splits, s)
                              : launch_decode_t<f16_t, 64, f16_t>(a, group, w, n_splits, s);
}

}  // namespace skv
