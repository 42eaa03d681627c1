// Exact fp32 chunk attention (no reduced-precision products anywhere).
//
// Computes, for each (b, t, h), softmax attention over the key set J(b, t) of
// fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA"
// (section Change: keys are the active prefix, the causal mask is cut to it) and of
// TensorRT-LLM PR #18973 "FA4 variable-length cross-attention" (section Description: packed
// K/V segments per batch element, padded Q).
//
// One wavefront per query row. Keys are visited in tiles of 64, one key per lane: the lane
// forms the fp32 dot product with the query (held in LDS and read by broadcast), the wave
// takes the tile maximum, rescales its running sum and output, and accumulates the output
// with each lane owning D/64 output columns. exp is the accurate expf. This path serves
// fp32 caches, which are small; the bf16/fp16 paths live in attn_flash.hip / attn_decode.hip.
#include "common.h"

namespace skv {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D, typename OutT>
__global__ void __launch_bounds__(256) k_attn_f32(AttnArgs a) {
  constexpr int kWaves = 4;
  constexpr int kPer = D / 64;  // output columns per lane
  __shared__ float q_lds[kWaves][D];
  __shared__ float p_lds[kWaves][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;  // ((b * Tq + t) * Hq + h)
  const int64_t rows = (int64_t)a.B * a.Tq * a.Hq;
  if (row >= rows) return;  // no block-level barrier below: waves are independent
  const int h = (int)(row % a.Hq);
  const int t = (int)((row / a.Hq) % a.Tq);
  const int b = (int)(row / ((int64_t)a.Hq * a.Tq));
  const int g = h / (a.Hq / a.Hkv);

  const float* q = (const float*)a.q + row * D;
  OutT* out = (OutT*)a.out + row * D;
  const KeySet ks = key_set(a, b);
  if (!ks.ok) {
    for (int i = 0; i < kPer; ++i) out[lane + 64 * i] = from_f32<OutT>(0.f);
    if (a.lse && lane == 0) a.lse[((int64_t)b * a.Hq + h) * a.Tq + t] = -INFINITY;
    if (lane == 0 && t == 0 && h == 0) report(a.err, dev_error_bit(a));
    return;
  }
  for (int i = 0; i < kPer; ++i) q_lds[wave][lane + 64 * i] = q[lane + 64 * i];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  const float* kbase = (const float*)a.k;
  const float* vbase = (const float*)a.v;
  const int pos = ks.len - a.Tq + t;  // bottom-right aligned query position
  const int lim = row_limit(a.mask, a.block, pos, ks.len);  // last visible key
  const int end = ks.visit;
  float m = -INFINITY, l = 0.f;
  float o[kPer];
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;

  for (int j0 = 0; j0 < end; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= lim) {
      const float4* kr = (const float4*)(kbase + ((ks.base_row + j) * a.Hkv + g) * D);
      float acc = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4) {
        float4 kv = kr[d4];
        acc = fmaf(q_lds[wave][4 * d4 + 0], kv.x, acc);
        acc = fmaf(q_lds[wave][4 * d4 + 1], kv.y, acc);
        acc = fmaf(q_lds[wave][4 * d4 + 2], kv.z, acc);
        acc = fmaf(q_lds[wave][4 * d4 + 3], kv.w, acc);
      }
      s = acc * a.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -INFINITY) continue;  // nothing visible yet
    const float alpha = expf(m - m_new);  // m = -inf gives 0
    const float p = expf(s - m_new);      // s = -inf gives 0
    l = l * alpha + wave_sum(p);
    m = m_new;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    p_lds[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int i = 0; i < kPer; ++i) o[i] *= alpha;
    const int n = end - j0 < 64 ? end - j0 : 64;
    for (int jj = 0; jj < n; ++jj) {
      const float pj = p_lds[wave][jj];
      if (pj == 0.f) continue;  // hidden keys (and full-capacity tail rows) add nothing
      const float* vr = vbase + ((ks.base_row + j0 + jj) * a.Hkv + g) * D;
      for (int i = 0; i < kPer; ++i) o[i] = fmaf(pj, vr[lane + 64 * i], o[i]);
    }
  }
  const float inv = 1.f / l;
  for (int i = 0; i < kPer; ++i) out[lane + 64 * i] = from_f32<OutT>(o[i] * inv);
  if (a.lse && lane == 0) a.lse[((int64_t)b * a.Hq + h) * a.Tq + t] = m + logf(l);
}

hipError_t launch_attn_f32(const AttnArgs& a, int D, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Tq * a.Hq;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (D == 128) hipLaunchKernelGGL((k_attn_f32<128, float>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_attn_f32<64, float>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace skv
