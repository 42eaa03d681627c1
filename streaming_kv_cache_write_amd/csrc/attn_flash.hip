// Fused chunk attention for bf16/fp16 caches on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T) V over the key set J(b, t): the active prefix of a slab or
// ring (fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA",
// section Change), a packed cu_seqlens_kv segment with padded Q (TensorRT-LLM PR #18973 "FA4
// variable-length cross-attention", section Description), or -- for the comparison arm -- all
// cap rows with the unpopulated tail masked (fish-speech #1312, section Problem). GQA heads map
// by index; nothing is expanded.
//
// Layout of the work (one workgroup = 4 wavefronts = 128 queries of one (b, h)):
//   * Each wavefront owns 32 queries. It computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_{bf16,f16}: A = a 32-key slice of the K tile (LDS), B = its queries
//     (registers, loaded once). In the 32x32 accumulator a lane holds one query column and 16
//     of the 32 keys, so the row max / row sum need only in-lane work plus one exchange with
//     lane^32.
//   * Online softmax in fp32 with exp2 and the scale folded into one FMA per score; masked
//     entries are selected to -inf (never multiplied), so a masked key contributes exactly 0.
//     The reference max moves (and O is rescaled) only when a tile's max passes it by more than
//     2^8 in probability; otherwise the rescale factor is exactly 1 and skipped. Row sums add
//     the rounded probabilities with dot2 instructions.
//   * O^T += V^T P^T with the same MFMA: P stays in registers (the accumulator's key order is
//     mapped onto the MFMA's k slots, and V^T is read from LDS in that same order).
//   * K/V tiles of 64 keys are staged in LDS (K rows padded by 16 bytes, V rows by 64 bytes,
//     so neither the K reads nor the transposed V reads conflict on the 64 banks); the next
//     tile's global loads are issued before the current tile's math.
//   * The two wavefronts sharing a SIMD (one from each of the CU's two workgroups) overlap
//     matrix-core and vector work: a wavefront raises its priority while it issues MFMAs, so
//     the other one's softmax fills the vector ALU meanwhile.
//   * Workgroup ids are remapped so the query tiles of one (b, h) run on the same XCD and
//     share its L2 copy of K/V (dispatch hands consecutive workgroup ids to the 8 XCDs in turn).
#include <type_traits>

#include "common.h"

namespace skv {

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<f16_t> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The running max used as the softmax reference moves only when a tile's max exceeds it by more
// than this many powers of two (after the log2(e) * scale fold). Until then the stale reference
// is kept: probabilities stay below 2^8, far inside bf16/fp16 range, O needs no rescale, and the
// final O / l and lse are unchanged because numerator and denominator share the reference.
constexpr float kRescaleLog2 = 8.f;

// s_waitcnt vmcnt(0) (gfx9 encoding; expcnt and lgkmcnt fields left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

// row sum of 8 probabilities as rounded for the P V product, by 4 dot2 with (1, 1)
__device__ __forceinline__ float sum8(bf16x8 p, float acc) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf2;
  const bf2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf2{p[2 * i], p[2 * i + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float sum8(f16x8 p, float acc) {
  typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2;
  const h2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(h2{p[2 * i], p[2 * i + 1]}, one, acc, false);
  return acc;
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle, range checked
// against num_records: out-of-range loads return zero).
constexpr int kBufferRsrcWord3 = 0x00020000;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename OutT> __device__ __forceinline__ void store4(OutT* p, float a, float b, float c,
                                                                float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c,
                                                          float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c,
                                                           float d) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4;
  *(v4*)p = v4{(bf16_t)a, (bf16_t)b, (bf16_t)c, (bf16_t)d};
}
template <> __device__ __forceinline__ void store4<f16_t>(f16_t* p, float a, float b, float c,
                                                          float d) {
  typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 v4;
  *(v4*)p = v4{(f16_t)a, (f16_t)b, (f16_t)c, (f16_t)d};
}

constexpr int kFlashBM = 128;  // queries per workgroup
constexpr int kFlashBN = 64;   // keys per tile

// PV16: run P V in fp16 (P rounded to fp16, V converted bf16 -> fp16 as it is staged in LDS)
// instead of the input type. Used for bf16 inputs with an fp32 output, where bf16-rounded P
// would be the dominant error of the result.
template <typename T, int D, typename OutT, bool PV16>
__global__ void __launch_bounds__(256, 2) k_attn_flash(AttnArgs a, int n_qtiles) {
  typedef typename Mfma<T>::vec vec;
  typedef typename std::conditional<PV16, f16_t, T>::type TV;  // type of V and P in P V
  typedef typename Mfma<TV>::vec vecv;
  constexpr int BN = kFlashBN;
  constexpr int LDK = D + 8;           // K row stride in LDS, elements (16-byte pad)
  constexpr int LDV = D + 32;          // V row stride: 64-byte pad. A row is then 16 dwords
                                       // (mod 64) on from the last, and the transposed read of
                                       // two 16-lane groups (4 rows x 2 x 32 bytes) hits 64
                                       // distinct banks
  constexpr int DC = D / 16;           // 16-wide d chunks of the QK^T contraction
  constexpr int DB = D / 32;           // 32-row d blocks of O^T
  constexpr int VPR = D / 8;           // 16-byte vectors per K/V row
  constexpr int LOADS = BN * VPR / 256;
  __shared__ __attribute__((aligned(16))) T Ks[2][BN * LDK];  // double-buffered tiles
  __shared__ __attribute__((aligned(16))) TV Vs[2][BN * LDV];

  // workgroup -> (query tile, head, batch element); tiles of one head stay on one XCD
  const int nb = gridDim.x, bid = blockIdx.x;
  const int full = nb & ~7;
  const int logical = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int qt = logical % n_qtiles;
  const int bh = logical / n_qtiles;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int my_q = qt * kFlashBM + wave * 32 + l32;
  const bool q_ok = my_q < a.Tq;
  OutT* out_row = (OutT*)a.out + (((int64_t)b * a.Tq + my_q) * a.Hq + h) * D;

  const KeySet ks = key_set(a, b);
  if (!ks.ok) {  // uniform over the workgroup
    if (q_ok)
      for (int d = 4 * hi; d < D; d += 8) store4<OutT>(out_row + d, 0.f, 0.f, 0.f, 0.f);
    if (q_ok && a.lse && hi == 0) a.lse[((int64_t)b * a.Hq + h) * a.Tq + my_q] = -INFINITY;
    if (tid == 0 && qt == 0 && h == 0) report(a.err, dev_error_bit(a));
    return;
  }

  // this wave's queries as the B operand of S^T = K Q^T (loaded once)
  vec qreg[DC];
  {
    const T* qp = (const T*)a.q + (((int64_t)b * a.Tq + my_q) * a.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (q_ok) qreg[c] = *(const vec*)(qp + 16 * c);
      else qreg[c] = vec{};
    }
    // Wait for these loads here, on every path. Otherwise the compiler may still count them as
    // outstanding at the head of the tile loop and wait there for all loads -- including the
    // next tile's, issued one step earlier to hide their latency.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // key range: the workgroup's last query bounds it; keys below key_full are visible to
  // every query of the workgroup, so those tiles need no mask at all
  const int q_first = qt * kFlashBM;
  const int q_last = min(q_first + kFlashBM, a.Tq) - 1;
  const int shift = ks.len - a.Tq;  // query t sits at absolute position t + shift
  const int key_end = a.full_cap ? ks.visit : row_limit(a.mask, a.block, q_last + shift, ks.len) + 1;
  const int key_full = row_limit(a.mask, a.block, q_first + shift, ks.len) + 1;
  const int my_lim = row_limit(a.mask, a.block, my_q + shift, ks.len);  // last key this row sees
  const int full_end = min(key_end, (key_full / BN) * BN);

  const int64_t rstride = (int64_t)a.Hkv * D;
  const T* kbase = (const T*)a.k + ks.base_row * rstride + (int64_t)g * D;
  const T* vbase = (const T*)a.v + ks.base_row * rstride + (int64_t)g * D;

  uint4 kr[LOADS], vr[LOADS];
  // Tile loads are buffer loads: a per-tile resource (uniform base = the tile's first row,
  // size = its rows that exist) plus a loop-invariant 32-bit lane offset. Rows past the end of
  // the visited range fall outside the resource and read as zero, so no load is branched,
  // predicated or followed by a zero fill, and no per-load address arithmetic is needed.
  uint32_t ld_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int idx = tid + 256 * i;
    ld_off[i] = (uint32_t)(((idx / VPR) * rstride + 8 * (idx % VPR)) * sizeof(T));
  }
  const int row_bytes = (int)(rstride * sizeof(T));
  auto load_tile = [&](int tile) {
    const int rows = min(ks.visit - tile, BN);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)tile * rstride), (short)0, rows * row_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)tile * rstride), (short)0, rows * row_bytes, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)ld_off[i], 0, 0);
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)ld_off[i], 0, 0);
      __builtin_memcpy(&kr[i], &a, 16);
      __builtin_memcpy(&vr[i], &c, 16);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + 256 * i;
      const int key = idx / VPR, c8 = idx % VPR;
      *(uint4*)&Ks[buf][key * LDK + 8 * c8] = kr[i];
      if constexpr (PV16 && !std::is_same<T, f16_t>::value) {
        const T* e = (const T*)&vr[i];
        typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 h8;
        h8 hv;
#pragma unroll
        for (int k = 0; k < 8; ++k) hv[k] = (f16_t)(float)e[k];
        *(h8*)&Vs[buf][key * LDV + 8 * c8] = hv;
      } else {
        *(uint4*)&Vs[buf][key * LDV + 8 * c8] = vr[i];
      }
    }
  };

  // transposed V reads: row and column offsets of this lane's 8-byte chunk (see the PV step)
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;

  // One 64-key tile held in LDS buffer `buf`: S^T = K Q^T, online softmax, O^T += V^T P^T;
  // meanwhile the next tile (already in registers) goes to the other buffer and the one after
  // it is fetched from HBM -- one workgroup barrier per tile.
  // MASKED selects the variant with the per-score visibility test; the two variants run in
  // separate loops so no branch sits between the S^T products and their use.
  auto step = [&](int tile, int buf, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const T* Kt = Ks[buf];
    const TV* Vt = Vs[buf];

    // s[sb][4i+j] = score(key tile+32sb+8i+4hi+j, query my_q)
    f32x16 s[2];
    __builtin_amdgcn_s_setprio(1);  // matrix-core phase: issue ahead of softmax waves
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) {
        const vec ka = *(const vec*)&Kt[(sb * 32 + l32) * LDK + 16 * cc + 8 * hi];
        s[sb] = Mfma<T>::mma(ka, qreg[cc], s[sb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    float sv[2][16];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = tile + 32 * sb + 8 * (r >> 2) + 4 * hi + (r & 3);
        sv[sb][r] = (!MASKED || key <= my_lim) ? s[sb][r] : -INFINITY;
      }
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv[sb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // (mt - m) is NaN when both are -inf (a row with nothing visible yet): no move
    const bool grow = (mt - m) * c > kRescaleLog2;
    const float m_new = grow ? mt : m;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);  // exactly 1 while the reference stays
    const float mc = m_use * c;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[sb][r] = fast_exp2(fmaf(sv[sb][r], c, -mc));
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }

    // P^T as B operands, one per 16-key chunk: k slot jj of lane half hi holds
    // key 4hi+jj (jj < 4) or 8+4hi+(jj-4) (jj >= 4) of the chunk. The row sum adds the
    // rounded values, the weights the product actually applies.
    vecv pb[4];
    float psum = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int sb = kc >> 1, r0 = 8 * (kc & 1);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[kc][jj] = (TV)sv[sb][r0 + jj];
      psum = sum8(pb[kc], psum);
    }
    lsum = lsum * alpha + psum;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // A operand V^T (32 d rows x 16 keys) by two transposed LDS reads: lane k of each
        // 16-lane group points at V[key0 + k/4][d0 + 4(k%4)], and lane i receives
        // V[key0 + t][d0 + i], t = 0..3 -- four keys of one d column. The keys are the MFMA
        // k slots 0..3 (keys 4hi+t of the chunk) and 4..7 (keys 8+4hi+t), the order P holds.
        const TV* vp = Vt + (16 * kc + 4 * hi + tr_row) * LDV + 32 * db + tr_col;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * LDV));
        vecv va;
        __builtin_memcpy(&va, &x0, 8);
        __builtin_memcpy((char*)&va + 8, &x1, 8);
        o[db] = Mfma<TV>::mma(va, pb[kc], o[db]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (tile + BN < key_end) {
      store_tile(buf ^ 1);  // nobody reads that buffer: every wave passed the last barrier
      if (tile + 2 * BN < key_end) load_tile(tile + 2 * BN);
    }
    __syncthreads();
  };

  if (key_end > 0) {
    load_tile(0);
    store_tile(0);
    if (BN < key_end) load_tile(BN);
    __syncthreads();
  }
  int tile = 0, buf = 0;
  for (; tile < full_end; tile += BN, buf ^= 1) step(tile, buf, std::false_type{});
  for (; tile < key_end; tile += BN, buf ^= 1) step(tile, buf, std::true_type{});

  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (q_ok) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * hi;
        store4<OutT>(out_row + d0, o[db][4 * i] * inv, o[db][4 * i + 1] * inv,
                     o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
      }
    if (a.lse && hi == 0) {
      const float mm = m == -INFINITY ? 0.f : m;
      a.lse[((int64_t)b * a.Hq + h) * a.Tq + my_q] = mm * a.scale + logf(ltot);
    }
  }
}

template <typename T, typename OutT>
static hipError_t launch_flash_t(const AttnArgs& a, int D, hipStream_t s) {
  constexpr bool kPV16 = std::is_same<T, bf16_t>::value && std::is_same<OutT, float>::value;
  const int n_qtiles = (a.Tq + kFlashBM - 1) / kFlashBM;
  const int64_t blocks = (int64_t)n_qtiles * a.Hq * a.B;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  if (D == 128)
    hipLaunchKernelGGL((k_attn_flash<T, 128, OutT, kPV16>), grid, block, 0, s, a, n_qtiles);
  else
    hipLaunchKernelGGL((k_attn_flash<T, 64, OutT, kPV16>), grid, block, 0, s, a, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_attn_flash(const AttnArgs& a, int dtype, int out_dtype, int D, hipStream_t s) {
  if (dtype == SKV_BF16)
    return out_dtype == SKV_F32 ? launch_flash_t<bf16_t, float>(a, D, s)
                                : launch_flash_t<bf16_t, bf16_t>(a, D, s);
  return out_dtype == SKV_F32 ? launch_flash_t<f16_t, float>(a, D, s)
                              : launch_flash_t<f16_t, f16_t>(a, D, s);
}

}  // namespace skv
