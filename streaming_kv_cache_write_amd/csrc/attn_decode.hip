// Decode-sized attention (Tq <= 4): split-K over the key range, then an LSE-weighted merge.
//
// Each decode step i attends its single new query to the active prefix kv_len = T + i + 1
// (fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA",
// section Change); the step reads 2*kv_len*Hkv*D*elem bytes of K/V and does almost no math
// per byte, so the kernel is built to stream K/V at HBM rate:
//   * one workgroup per (split, KV head, batch element); the key range [0, visit) is cut into
//     gridDim.x equal parts computed on the device from kv_len, so a fixed grid (graph replay
//     with a device kv_len) still spreads any length over every workgroup;
//   * all query rows of a GQA group (Hq/Hkv heads x Tq rows, <= 16) share each K/V load:
//     S = Q K^T on v_mfma_f32_16x16x32 (K straight from global memory in the B-operand
//     layout, the group's query rows as A), softmax in fp32, and P V on the vector ALUs with
//     P kept in fp32 (each lane owns 8 output columns of a quarter of the keys);
//   * a workgroup of 4 wavefronts takes one split; its wavefronts merge in LDS. With several
//     splits, each workgroup writes its unnormalised (m, l, o) to the caller's workspace and a
//     second launch merges them with weights exp(m_s - max m).
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

constexpr int kDecWaves = 4;  // wavefronts per workgroup; they share one split's tiles
// Per-lane merge state in the "row layout": row r0 + lane/16, columns [8*(lane%16), +8).
struct MergeState {
  float M, L, o[8];
};

__device__ __forceinline__ void merge_init(MergeState& st) {
  st.M = -INFINITY;
  st.L = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = 0.f;
}

// Fold a partial (m, l, o) into st with weights exp2((m - M) * c2) (online, max-safe).
__device__ __forceinline__ void merge_add(MergeState& st, float m, float l, const float* o,
                                          float c2) {
  const float m_new = fmaxf(st.M, m);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float wa = __builtin_amdgcn_exp2f((st.M - m_use) * c2);
  const float wb = __builtin_amdgcn_exp2f((m - m_use) * c2);
  st.L = st.L * wa + l * wb;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = st.o[e] * wa + o[e] * wb;
  st.M = m_new;
}

// LDS staging of one state per (wavefront, row): m, l and D output columns.
template <int D, int NR>
struct DecStage {
  float m[kDecWaves][NR];
  float l[kDecWaves][NR];
  float o[kDecWaves][NR][D];
};

// Combine the kDecWaves staged states of row r, columns [8dc, 8dc+8).
template <int D, int NR>
__device__ __forceinline__ void combine_staged(const DecStage<D, NR>& sg, int r, int dc,
                                               float c2, MergeState& st) {
  merge_init(st);
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = dc < D / 8 ? sg.o[w][r][8 * dc + e] : 0.f;
    merge_add(st, sg.m[w][r], sg.l[w][r], o, c2);
  }
}

template <typename OutT>
__device__ __forceinline__ void write_row(const AttnArgs& a, int D, int group, int b, int g, int r,
                                          int dc, const MergeState& st) {
  const int t = r / group, h = g * group + (r - t * group);
  const float inv = st.L > 0.f ? 1.f / st.L : 0.f;  // L = 0: the batch element was rejected
  if (dc < D / 8) {
    OutT* out = (OutT*)a.out + (((int64_t)b * a.Tq + t) * a.Hq + h) * D + 8 * dc;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = from_f32<OutT>(st.o[e] * inv);
  }
  if (a.lse && dc == 0)
    a.lse[((int64_t)b * a.Hq + h) * a.Tq + t] = st.L > 0.f ? st.M * a.scale + logf(st.L) : -INFINITY;
}

// The workgroup merges the n_splits partials of the R rows of (b, g) and writes the outputs:
// wavefront w folds splits w, w + kDecWaves, ... (loads of 8 splits at a time, nothing
// branching on loaded data), then wavefront 0 combines the kDecWaves states through LDS.
template <int D, int NR, typename OutT>
__device__ __forceinline__ void merge_splits(const AttnArgs& a, int group, const float* ws_o,
                                             const float* ws_ml, DecStage<D, NR>& sg, int b, int g,
                                             int n_splits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dc = lane & 15;
  const bool dc_ok = dc < D / 8;
  const int R = a.Tq * group;
  const float c2 = a.scale_log2;
    for (int r0 = 0; r0 < NR; r0 += 4) {
      const int r = r0 + (lane >> 4);
      const bool row_ok = r < R;
      const size_t p0 = dec_part_index(b, g, row_ok ? r : 0, 0, a.Hkv, n_splits);
      MergeState st;
      merge_init(st);
      constexpr int kBatch = 8;
      for (int s0 = wave; s0 < n_splits; s0 += kBatch * kDecWaves) {
        float2 ml[kBatch];
        float4 oa[kBatch], ob[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int sp = s0 + u * kDecWaves;
          const bool ok = sp < n_splits;
          ml[u] = ok ? *(const float2*)(ws_ml + 2 * (p0 + sp)) : make_float2(-INFINITY, 0.f);
          const float* po = ws_o + (p0 + (ok ? sp : 0)) * D + 8 * dc;
          oa[u] = (ok && dc_ok) ? *(const float4*)po : make_float4(0.f, 0.f, 0.f, 0.f);
          ob[u] = (ok && dc_ok) ? *(const float4*)(po + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float o8[8] = {oa[u].x, oa[u].y, oa[u].z, oa[u].w, ob[u].x, ob[u].y, ob[u].z, ob[u].w};
          merge_add(st, ml[u].x, ml[u].y, o8, c2);
        }
      }
      __syncthreads();  // the previous pass's reads of the staging area are done
      if (row_ok) {
        if (dc == 0) {
          sg.m[wave][r] = st.M;
          sg.l[wave][r] = st.L;
        }
        if (dc_ok)
#pragma unroll
          for (int e = 0; e < 8; ++e) sg.o[wave][r][8 * dc + e] = st.o[e];
      }
      __syncthreads();
      if (wave == 0 && row_ok) {
        MergeState fin;
        combine_staged<D, NR>(sg, r, dc, c2, fin);
        write_row<OutT>(a, D, group, b, g, r, dc, fin);
      }
    }
}

// NR: query rows per KV head rounded up to 4, 8 or 16 (R = Tq * Hq/Hkv <= NR).
// Workgroup = kDecWaves wavefronts per (split, KV head g, batch element b); the split's key
// range is cut into 64-key tiles dealt round-robin to the wavefronts. Each wavefront keeps its
// own online-softmax state; the workgroup merges them in LDS. With one split that is the
// output; otherwise the workgroup's partial goes to the workspace and k_decode_merge, a second
// launch, merges the splits. (Merging in this launch, by the last workgroup to arrive, needs a
// release fence per workgroup -- an L2 write-back on this multi-XCD chip -- and measured slower
// than the second launch at every length tried, 64 to 32768 keys.)
// FUSED: one launch per decode step with the write cursor on the device (attn_decode_step):
// c = *cursor; the new rows k_new/v_new [B, Tq, Hkv, D] are written to cache rows c .. c+Tq-1
// and attended over as keys c .. c+Tq-1 straight from the sources (no wavefront of this launch
// reads a cache row another one writes); the last (b, g) to finish sets *cursor = c+Tq and
// kv_len_out[:] = c+Tq, after every wavefront has read the cursor.
template <typename T, int D, int NR, typename OutT, bool FUSED>
__global__ void __launch_bounds__(64 * kDecWaves) k_attn_decode(AttnArgs a, int group, float* ws,
                                                                int n_splits) {
  typedef typename Mfma16<T>::vec vec;
  constexpr int DQ = D / 32;  // 32-wide d chunks of the QK^T contraction
  __shared__ __attribute__((aligned(16))) float P[kDecWaves][kDecBN][kDecRows];
  __shared__ float alpha_s[kDecWaves][kDecRows];
  __shared__ __attribute__((aligned(16))) DecStage<D, NR> sg;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
    if (!fits && threadIdx.x == 0 && split == 0 && g == 0 && b == 0) report(a.err, SKV_DEV_CURSOR_FULL);
  } else {
    ks = key_set(a, b);
    if (!ks.ok && threadIdx.x == 0 && split == 0 && g == 0) report(a.err, dev_error_bit(a));
  }
  // this split's share of the visited rows, in whole 64-key tiles
  int per = (ks.visit + n_splits - 1) / n_splits;
  per = (per + kDecBN - 1) & ~(kDecBN - 1);
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
    if (split == 0 && wave == 0 && ks.ok) {  // this head's slice of the new rows goes into the cache
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
  float (*Pw)[kDecRows] = P[wave];

  // the wavefronts of the workgroup take the split's tiles in turn; no workgroup barrier in
  // here (trip counts differ): P and alpha_s are per wavefront
  for (int tile = start + kDecBN * wave; tile < end; tile += kDecBN * kDecWaves) {
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
      *(float4*)&Pw[16 * kb + col][4 * quad] = make_float4(s[kb][0], s[kb][1], s[kb][2], s[kb][3]);
    if (col == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) alpha_s[wave][4 * quad + j] = alpha[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float al = alpha_s[wave][r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v[8];
      unpack8<T>(vraw[i], v);
      const float* pr = Pw[kg + 4 * i];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float p = pr[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, v[e], acc[r][e]);
      }
    }
    // P and alpha_s are rewritten by the next tile of this wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  // stage this wavefront's state, then merge the workgroup's wavefronts row by row
  if (col == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * quad + j < NR) {
        sg.m[wave][4 * quad + j] = m[j];
        sg.l[wave][4 * quad + j] = l[j];
      }
  if (kg == 0 && dc_ok)
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) sg.o[wave][r][8 * dc + e] = acc[r][e];
  __syncthreads();

  if (n_splits == 1) {  // the workgroup saw every key: its merge is the output
    if (wave == 0)
      for (int r0 = 0; r0 < R; r0 += 4) {
        const int r = r0 + (lane >> 4);
        MergeState st;
        if (r < R) {
          combine_staged<D, NR>(sg, r, dc, c2, st);
          write_row<OutT>(a, D, group, b, g, r, dc, st);
        }
      }
  } else {
    // the workgroup's partial goes to the workspace
    if (wave == 0)
      for (int r0 = 0; r0 < R; r0 += 4) {
        const int r = r0 + (lane >> 4);
        if (r >= R) continue;
        MergeState st;
        combine_staged<D, NR>(sg, r, dc, c2, st);
        const size_t pi = dec_part_index(b, g, r, split, a.Hkv, n_splits);
        if (dc_ok) {
          float* po = ws_o + pi * D + 8 * dc;
          *(float4*)po = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
          *(float4*)(po + 4) = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
        }
        if (dc == 0) *(float2*)(ws_ml + 2 * pi) = make_float2(st.M, st.L);
      }
    return;  // k_decode_merge finishes the step
  }
  if constexpr (FUSED) {
    // one split per (b, g): every workgroup of the launch read the cursor before it got here,
    // so the last one to finish may move it (an arrival count only; no data is handed over)
    if (threadIdx.x == 0) {
      const int old = __hip_atomic_fetch_add(&counters[a.B * a.Hkv], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old == a.B * a.Hkv - 1) {
        if (ks.ok) {
          if (a.kv_len_out)
            for (int bb = 0; bb < a.B; ++bb) a.kv_len_out[bb] = cur + a.Tq;
          *a.cursor = cur + a.Tq;
        }
        __hip_atomic_store(&counters[a.B * a.Hkv], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Second launch of the two-kernel variant: one workgroup per (b, KV head) merges the splits.
// In the fused step, workgroup (0, 0) also moves the cursor: every workgroup of the first
// launch read it before this launch started, and no workgroup of this one reads it otherwise.
template <int D, int NR, typename OutT, bool FUSED>
__global__ void __launch_bounds__(64 * kDecWaves) k_decode_merge(AttnArgs a, int group, float* ws,
                                                                 int n_splits) {
  __shared__ __attribute__((aligned(16))) DecStage<D, NR> sg;
  const int g = blockIdx.x, b = blockIdx.y;
  const float* ws_o = ws + dec_counter_floats(a.B, a.Hkv);
  const float* ws_ml = ws_o + dec_o_floats(a.B, a.Hkv, D, n_splits);
  merge_splits<D, NR, OutT>(a, group, ws_o, ws_ml, sg, b, g, n_splits);
  if constexpr (FUSED) {
    if (b == 0 && g == 0 && threadIdx.x == 0) {
      const int cur = *a.cursor;
      if (cur >= 0 && (int64_t)cur + a.Tq <= a.cap) {
        if (a.kv_len_out)
          for (int bb = 0; bb < a.B; ++bb) a.kv_len_out[bb] = cur + a.Tq;
        *a.cursor = cur + a.Tq;
      }
    }
  }
}

// Split count used by both the launcher and the workspace query.
int decode_splits(int B, int Hkv, int max_len) {
  const int tiles = (max_len + kDecBN - 1) / kDecBN;
  const int by_tiles = (tiles + kDecWaves - 1) / kDecWaves;  // one tile per wavefront at most
  int target = 2048 / (B * Hkv * kDecWaves);  // about two wavefronts per SIMD over the chip
  if (target < 1) target = 1;
  int s = by_tiles < target ? by_tiles : target;
  return s < 1 ? 1 : s;
}

size_t decode_workspace_bytes(int B, int Hkv, int D, int n_splits) {
  return (dec_counter_floats(B, Hkv) + dec_o_floats(B, Hkv, D, n_splits) +
          dec_ml_floats(B, Hkv, n_splits)) * sizeof(float);
}

template <typename T, int D, int NR, typename OutT, bool FUSED>
static hipError_t launch_decode_nr(const AttnArgs& a, int group, float* ws, int n_splits,
                                   hipStream_t s) {
  dim3 grid(n_splits, a.Hkv, a.B), block(64 * kDecWaves);
  hipLaunchKernelGGL((k_attn_decode<T, D, NR, OutT, FUSED>), grid, block, 0, s, a, group, ws, n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  hipLaunchKernelGGL((k_decode_merge<D, NR, OutT, FUSED>), dim3(a.Hkv, a.B), block, 0, s, a, group, ws,
                     n_splits);
  return hipGetLastError();
}

template <typename T, int D, typename OutT, bool FUSED>
static hipError_t launch_decode_f(const AttnArgs& a, int group, float* ws, int n_splits,
                                  hipStream_t s) {
  const int R = a.Tq * group;
  if (R <= 4) return launch_decode_nr<T, D, 4, OutT, FUSED>(a, group, ws, n_splits, s);
  if (R <= 8) return launch_decode_nr<T, D, 8, OutT, FUSED>(a, group, ws, n_splits, s);
  return launch_decode_nr<T, D, 16, OutT, FUSED>(a, group, ws, n_splits, s);
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
