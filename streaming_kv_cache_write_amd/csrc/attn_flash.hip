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
//     lane^32 (v_permlane32_swap).
//   * Online softmax in fp32 with exp2 and the scale folded into one FMA per score; masked
//     entries are selected to -inf (never multiplied), so a masked key contributes exactly 0.
//     The reference max moves (and O is rescaled) only when a tile's max passes it by more than
//     2^8 in probability; otherwise the rescale factor is exactly 1 and skipped. Row sums add
//     the rounded probabilities with dot2 instructions.
//   * O^T += V^T P^T with the same MFMA: P stays in registers (the accumulator's key order is
//     mapped onto the MFMA's k slots, and V^T is read from LDS in that same order by
//     transposed reads, ds_read_b64_tr_b16).
//   * K/V tiles of 64 keys go from HBM straight into LDS (buffer loads with the lds bit, no
//     registers in between); 16-byte granules are XOR-swizzled per row so the K reads and the
//     transposed V reads are free of bank conflicts without padding.
//   * Software pipeline, one workgroup barrier per tile: K runs one tile ahead of V. While
//     tile j's softmax runs on the vector ALUs, S^T of tile j+1 is computed on the matrix
//     cores -- the two streams are interleaved instruction by instruction (scheduling group
//     barriers), since a wavefront issues in order -- and the loads of V(j+1) and K(j+2) are in
//     flight. Buffers alternate by tile parity (the loop is unrolled by two), so every LDS
//     offset is an immediate and the compiler sees that a load into one buffer cannot alias
//     reads of the other.
//   * Workgroup ids are remapped so the query tiles of one (b, h) run on the same XCD and
//     share its L2 copy of K/V (dispatch hands consecutive workgroup ids to the 8 XCDs in turn),
//     with the (b, h) pairs dealt round-robin over the XCDs so unequal heads stay balanced.
//   * Q and O cross global memory as whole rows: Q goes straight into LDS like a K tile (in
//     the two tile buffers idle until tile 1) and is read from there once in the operand
//     layout; each wavefront's normalised output block is staged in an idle tile buffer and
//     stored 4 rows per instruction (the operand and accumulator layouts would touch 32 rows
//     per instruction).
//   * Tail split (optional, needs a workspace): when the last round of workgroups would leave
//     many of the CU slots idle, the items of that round are cut by key range into a few
//     pieces. Each piece stores its unnormalised O^T, reference max and row sums; the last
//     piece of an item to finish (an arrival count) merges them and writes the output.
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

// Workgroup barrier over LDS only: the wavefront's LDS operations have completed, while its
// global loads and stores stay in flight (__syncthreads would also drain those).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
constexpr int kFlashSlotsPerXcd = 64;  // 32 CUs x 2 resident workgroups
constexpr int kFlashMinPieceTiles = 16;  // a key-range piece covers at least this many tiles

// Which item (query tile, b, h) and key-range piece a workgroup runs. With the (b, h) pairs
// dealt evenly over the 8 XCDs each XCD runs items 0 .. nf + r - 1 of its own; items below nf
// run whole, the last r are each cut into `parts` key-range pieces (part-major order, so the
// pieces that read the same keys run together). parts == 1: no split (nf and r unused).
struct FlashGrid {
  int n_qtiles;
  int nf, r, parts;
  float* ws;  // parts > 1: arrival counters, then the pieces' partials
};

// Workspace of the tail split: the shared counter area (one int32 arrival counter per split
// item, at most 8 x 63, left at zero by every launch), then per (split item, piece) a block of
// 256 lanes x (D/2 floats of O^T + the reference max + the row sum), lane-interleaved.
__host__ __device__ constexpr int flash_piece_floats(int D) { return 256 * (D / 2 + 2); }
__host__ __device__ constexpr int flash_counter_floats(int) { return kWsCounterInts; }

// Device-coherent (sc1) buffer accesses, as agent-scope atomic stores and loads take: the
// pieces of one item run on one XCD, but nothing ties a later launch reusing the workspace to
// that XCD, so the partials bypass the per-XCD L2 state the same way the decode merge does.
constexpr int kFlashCoherent = 16;

// PV16: run P V in fp16 (P rounded to fp16, V converted bf16 -> fp16 in LDS after it lands)
// instead of the input type. Used for bf16 inputs with an fp32 output, where bf16-rounded P
// would be the dominant error of the result.
template <typename T, int D, typename OutT, bool PV16>
__global__ void __launch_bounds__(256, 2) k_attn_flash(AttnArgs a, FlashGrid fg) {
  typedef typename Mfma<T>::vec vec;
  typedef typename std::conditional<PV16, f16_t, T>::type TV;  // type of V and P in P V
  typedef typename Mfma<TV>::vec vecv;
  constexpr int BN = kFlashBN;
  constexpr int ROWB = D * 2;              // bytes per K/V row in LDS (no padding)
  constexpr int GPR = D / 8;               // 16-byte granules per row
  constexpr int RP256 = 256 / ROWB;        // rows per 256 bytes (one pass over the 64 banks)
  constexpr int TILE = BN * ROWB;          // bytes per K or V tile
  constexpr int CHUNKS = TILE / 1024;      // 1 KB pieces a wavefront's direct load fills
  constexpr int CPW = CHUNKS / 4;          // ... per wavefront and tile
  constexpr int RPC = 1024 / ROWB;         // rows per piece
  constexpr int DC = D / 16;               // 16-wide d chunks of the QK^T contraction
  constexpr int DB = D / 32;               // 32-row d blocks of O^T
  static_assert(CPW >= 1, "tile too small for four wavefronts");
  // Tiles land in LDS straight from global memory (buffer_load ... lds: 16 bytes per lane,
  // a wavefront fills 1 KB of consecutive bytes per instruction), so rows cannot be padded.
  // Instead the 16-byte granules of a row are XOR-swizzled: granule g of row r sits at
  // position g ^ sk(r) (K) or g ^ sv(r) (V), chosen so that the K reads (16 rows, one granule
  // each) and the transposed V reads (4 rows x 4 granules per half-wavefront) hit distinct
  // banks. The loading lane picks the global granule that belongs at its LDS position.
  // four separate LDS objects (not one array of buffers): the compiler then sees that a
  // direct load into one buffer cannot alias reads of another and adds no wait for it
  __shared__ __attribute__((aligned(1024))) unsigned char Ks0[TILE], Ks1[TILE], Vs0[TILE], Vs1[TILE];
  unsigned char* const Ks[2] = {Ks0, Ks1};
  unsigned char* const Vs[2] = {Vs0, Vs1};
  auto sk = [](int r) { return (r / RP256) % GPR; };
  auto sv = [](int r) { return 4 * ((r / RP256) % (GPR / 4)); };

  // workgroup -> (query tile, head, batch element). Dispatch deals consecutive workgroup ids
  // to the 8 XCDs in turn; the (b, h) pairs are dealt to the XCDs the same way (XCD x takes
  // bh = x, x + 8, ...), each with all its query tiles in order, so a head's K/V is shared in
  // one L2 and heads of unequal cost (ragged batch elements) spread over every XCD.
  // Every kernel argument in one batch of scalar loads and one wait (left to itself the
  // compiler loads each where it is first used: three dependent round trips before the first
  // query loads go out). The asm takes them all as inputs and passes the tile count through to
  // the mapping below; it is not volatile and touches no memory, so the metadata reads after
  // it stay scalar loads.
  int n_qtiles = fg.n_qtiles;
  asm("" : "+s"(n_qtiles) : "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.out), "s"(a.lse), "s"(a.kv_len_dev), "s"(a.cu),
      "s"(a.err), "s"(fg.ws), "s"(fg.nf), "s"(fg.r), "s"(fg.parts));
  asm("" : "+s"(n_qtiles) : "s"(a.B), "s"(a.Tq), "s"(a.Hq), "s"(a.Hkv), "s"(a.cap), "s"(a.kv_len_host),
      "s"(a.mask), "s"(a.block), "s"(a.full_cap), "s"(a.scale), "s"(a.scale_log2), "s"(gridDim.x));
  const int bid = blockIdx.x, BH = a.B * a.Hq;
  int qt, bh, part = 0, split_id = -1;
  if ((BH & 7) == 0) {
    int k = bid >> 3;
    if (fg.parts > 1 && k >= fg.nf) {  // piece `part` of item nf + ri
      const int u = k - fg.nf;
      part = u / fg.r;
      const int ri = u - part * fg.r;
      split_id = (bid & 7) * fg.r + ri;
      k = fg.nf + ri;
    }
    const int hl = k / n_qtiles;
    qt = k - hl * n_qtiles;
    bh = (bid & 7) + 8 * hl;
  } else {  // contiguous ranges of the (bh, qt) order per XCD
    const int full = gridDim.x & ~7;
    const int logical = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
    qt = logical % n_qtiles;
    bh = logical / n_qtiles;
  }
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;

  // (the wavefront index as a scalar: the buffer resources built from it stay in scalar
  // registers, with no loop over distinct per-lane values around each load and store)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int my_q = qt * kFlashBM + wave * 32 + l32;
  const bool q_ok = my_q < a.Tq;
  const int q0 = qt * kFlashBM + wave * 32;  // first query row of this wavefront
  const int n_qrows = __builtin_amdgcn_readfirstlane(max(min(32, a.Tq - q0), 0));  // (scalar)

  // This wave's 32 queries, the B operand of S^T = K Q^T, go from global memory straight into
  // LDS (Ks1 holds the rows of waves 0-1, Vs1 those of waves 2-3; both are idle until tile 1's
  // loads), laid out and swizzled like a K tile, and are read from there once in the operand
  // layout. Rows past Tq lie outside the load resource's range and read as zeros.
  const int row_stride = a.Hq * D * (int)sizeof(T);  // host-checked: 32 rows fit an int
  constexpr int QP = 32 * ROWB / 1024;  // 1 KB pieces of a wavefront's query rows
  unsigned char* const q_lds = (wave < 2 ? Ks1 : Vs1) + (wave & 1) * 32 * ROWB;
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const T*)a.q + (((int64_t)b * a.Tq + q0) * a.Hq + h) * D), (short)0,
        n_qrows > 0 ? (n_qrows - 1) * row_stride + D * (int)sizeof(T) : 0, kBufferRsrcWord3);
#pragma unroll
    for (int pc = 0; pc < QP; ++pc) {
      const int r = pc * RPC + lane / GPR;  // row of the wave's 32; (wave & 1) * 32 + r in the buffer
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void*)(q_lds + pc * 1024), 16,
          (int)(r * row_stride + 16 * ((lane % GPR) ^ sk((wave & 1) * 32 + r))), 0, 0, 0);
    }
  }

  vec qreg[DC];

  // An invalid length (reported once per launch) leaves the workgroup no tiles: it runs the
  // same path as an empty key set and writes zero rows with lse = -inf.
  const KeySet ks = key_set(a, b);
  if (!ks.ok && tid == 0 && qt == 0 && h == 0) report(a.err, dev_error_bit(a));

  // key range: the workgroup's last query bounds it; keys below key_full are visible to
  // every query of the workgroup, so those tiles need no mask at all
  const int q_first = qt * kFlashBM;
  const int q_last = min(q_first + kFlashBM, a.Tq) - 1;
  const int shift = ks.len - a.Tq;  // query t sits at absolute position t + shift
  const int key_end = a.full_cap ? ks.visit : row_limit(a.mask, a.block, q_last + shift, ks.len) + 1;
  const int key_full = row_limit(a.mask, a.block, q_first + shift, ks.len) + 1;
  int my_lim = row_limit(a.mask, a.block, my_q + shift, ks.len);  // last key this row sees
  int n_tiles = ks.ok ? (key_end + BN - 1) / BN : 0;
  int n_full = min(key_end, (key_full / BN) * BN) / BN;
  const int64_t rstride = (int64_t)a.Hkv * D;
  const T* kbase = (const T*)a.k + ks.base_row * rstride + (int64_t)g * D;
  const T* vbase = (const T*)a.v + ks.base_row * rstride + (int64_t)g * D;
  const int row_bytes = (int)(rstride * sizeof(T));
  int visit = ks.visit;  // rows from the tile base that exist
  if (split_id >= 0) {
    // this piece's tiles [t0, t1): everything below is re-based to tile t0
    const int t0 = part * n_tiles / fg.parts, t1 = (part + 1) * n_tiles / fg.parts;
    kbase += (int64_t)t0 * BN * rstride;
    vbase += (int64_t)t0 * BN * rstride;
    visit -= t0 * BN;
    my_lim -= t0 * BN;
    n_full = min(max(n_full - t0, 0), t1 - t0);
    n_tiles = t1 - t0;
  }

  // Direct loads: piece c = wave * CPW + i of a tile covers rows [c * RPC, +RPC); lane L fills
  // LDS bytes [c * 1024 + 16 L, +16), i.e. row c * RPC + L / GPR at position L % GPR, and so
  // loads global granule (L % GPR) ^ swizzle(row). Offsets are loop-invariant; the per-tile
  // resource (base = the tile's first row, size = its rows that exist) turns rows past the
  // visited range into zeros.
  uint32_t koff[CPW], voff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (wave * CPW + i) * RPC + lane / GPR, p = lane % GPR;
    koff[i] = (uint32_t)(r * row_bytes + 16 * (p ^ sk(r)));
    voff[i] = (uint32_t)(r * row_bytes + 16 * (p ^ sv(r)));
  }
  auto dma = [&](const T* base, int tile, unsigned char* dst, const uint32_t* off) {
    const int rows = min(visit - tile, BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (int64_t)tile * rstride), (short)0, rows * row_bytes, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < CPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (wave * CPW + i) * 1024), 16,
          (int)off[i], 0, 0, 0);
  };
  // PV16: this thread converts, in place, the V granules its own direct loads wrote (its loads
  // are complete once its vmcnt drains; the workgroup barrier then publishes the result)
  auto convert_v = [&](unsigned char* dst) {
    if constexpr (PV16) {
      typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 h8;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        unsigned char* pp = dst + (wave * CPW + i) * 1024 + 16 * lane;
        const bf16x8 x = *(const bf16x8*)pp;
        h8 y;
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = (f16_t)(float)x[k];
        *(h8*)pp = y;
      }
    }
  };

  // LDS read addresses. K (A operand of S^T): row sb*32 + l32, granule 2cc + hi -> position
  // (2cc + hi) ^ sk(row); sk is the same for sb = 0, 1. V^T (transposed reads, see the PV
  // step): row 16kc + 4hi + (lane%16)/4 (+8), column 32db + tr_col; the swizzle sv of these
  // rows depends on the lane only.
  const int swk = sk(l32);
  uint32_t kaddr[DC];
#pragma unroll
  for (int cc = 0; cc < DC; ++cc) kaddr[cc] = l32 * ROWB + 16 * ((2 * cc + hi) ^ swk);
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vrow = 4 * hi + tr_row;
  const int swv = sv(vrow);
  uint32_t vaddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vaddr[db] = vrow * ROWB + 16 * ((4 * db + tr_col / 8) ^ swv) + 2 * (tr_col % 8);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;
  f32x16 sacc[2][2];  // S^T of the current and the next tile (ping-pong by tile parity)

  // S^T = K Q^T for the tile in K buffer kb: s[sb][4i+j] = score(key 32sb+8i+4hi+j, my_q)
  auto qk = [&](int kb, f32x16* s) {
    const unsigned char* Kt = Ks[kb];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < DC; ++cc) {
        const vec ka = *(const vec*)(Kt + sb * 32 * ROWB + kaddr[cc]);
        s[sb] = Mfma<T>::mma(ka, qreg[cc], s[sb]);
      }
    }
  };

  // One tile j (parity P): V of tile j is in Vs[P], K of tile j + 1 in Ks[P ^ 1]. Issue the
  // direct loads of V(j+1) -> Vs[P^1] and K(j+2) -> Ks[P] (both buffers were last read before
  // the previous barrier), compute S^T of tile j + 1 while the softmax of tile j runs, then
  // O^T += V^T P^T, wait for this tile's loads and pass the workgroup barrier.
  auto step = [&](int j, auto parity) {
    constexpr int P = decltype(parity)::value;
    __builtin_amdgcn_sched_barrier(0);
    const int tile = j * BN;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) dma(vbase, tile + BN, Vs[P ^ 1], voff);
    if (j + 2 < n_tiles) dma(kbase, tile + 2 * BN, Ks[P], koff);

    f32x16* s = sacc[P];
    float sv_[2][16];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv_[sb][r] = s[sb][r];
    if (j >= n_full) {  // diagonal tiles only (uniform branch)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = tile + 32 * sb + 8 * (r >> 2) + 4 * hi + (r & 3);
          sv_[sb][r] = key <= my_lim ? sv_[sb][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv_[sb][r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max with lane ^ 32
    }
    // (mt - m) is NaN when both are -inf (a row with nothing visible yet): no move
    const bool grow = (mt - m) * c > kRescaleLog2;
    const float m_new = grow ? mt : m;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);  // exactly 1 while the reference stays
    const float mc = m_use * c;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }

    // One block from here to the barrier: S^T of the next tile on the matrix cores while this
    // tile's exponentials run on the vector ALUs, then O^T += V^T P^T. (The next tile's S^T is
    // computed even past the last tile, from whatever the buffer holds, and unused then: a
    // branch would split the block.)
    qk(P ^ 1, sacc[P ^ 1]);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv_[sb][r] = fast_exp2(fmaf(sv_[sb][r], c, -mc));
    // P^T as B operands, one per 16-key chunk: k slot jj of lane half hi holds
    // key 4hi+jj (jj < 4) or 8+4hi+(jj-4) (jj >= 4) of the chunk. The row sum adds the
    // rounded values, the weights the product actually applies.
    vecv pb[4];
    float psum = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int sb = kc >> 1, r0 = 8 * (kc & 1);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[kc][jj] = (TV)sv_[sb][r0 + jj];
      psum = sum8(pb[kc], psum);
    }
    lsum = lsum * alpha + psum;

    __builtin_amdgcn_s_setprio(1);
    const unsigned char* Vt = Vs[P];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // A operand V^T (32 d rows x 16 keys) by two transposed LDS reads: lane k of each
        // 16-lane group points at V[key0 + k/4][d0 + 4(k%4)], and lane i receives
        // V[key0 + t][d0 + i], t = 0..3 -- four keys of one d column. The keys are the MFMA
        // k slots 0..3 (keys 4hi+t of the chunk) and 4..7 (keys 8+4hi+t), the order P holds.
        const unsigned char* vp = Vt + 16 * kc * ROWB + vaddr[db];
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * ROWB));
        vecv va;
        __builtin_memcpy(&va, &x0, 8);
        __builtin_memcpy((char*)&va + 8, &x1, 8);
        o[db] = Mfma<TV>::mma(va, pb[kc], o[db]);
      }
    }
    // order within the block: each K read + S^T MFMA followed by softmax work, then the
    // transposed V reads and P V MFMAs
#pragma unroll
    for (int i = 0; i < 2 * DC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read (K)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA (S^T)
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // vector ALU (softmax)
    }
    // transposed V reads run three MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA (P V)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two transposed V reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this thread's direct loads have landed
    if (has_next) convert_v(Vs[P ^ 1]);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  if (n_tiles > 0) {
    dma(kbase, 0, Ks[0], koff);
    dma(vbase, 0, Vs[0], voff);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the query rows and the first K/V tiles have landed
  // Q in the operand layout: lane (l32, hi) of register c takes granule 2c + hi of row l32
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qreg[c] = *(const vec*)(q_lds + l32 * ROWB + 16 * ((2 * c + hi) ^ sk((wave & 1) * 32 + l32)));
  if (n_tiles > 0) convert_v(Vs[0]);
  lds_barrier();  // every wave holds its queries (Ks1 and Vs1 are free) and V(0) is converted
  if (n_tiles > 1) dma(kbase, BN, Ks[1], koff);
  if (n_tiles > 0) qk(0, sacc[0]);
  // K(1) has landed and every wave has read Ks[0] before tile 0's step refills it; nothing is
  // outstanding at the head of the tile loop, where a wait would also cover the next tiles'
  // loads
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  int j = 0;
  for (; j + 2 <= n_tiles; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < n_tiles) step(j, std::integral_constant<int, 0>{});

  if (split_id >= 0) {
    // Store this piece's partial; the last piece of the item to arrive merges all of them.
    const int PF = flash_piece_floats(D);
    float* const blocks = fg.ws + flash_counter_floats(8 * fg.r) + (size_t)split_id * fg.parts * PF;
    auto rsrc = [&](int p) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(blocks + (size_t)p * PF), (short)0,
                                               PF * (int)sizeof(float), kBufferRsrcWord3);
    };
    // float offset of lane data: O^T group gi (db = gi / 4, rows 4i .. 4i+3 of the 16) as one
    // float4 per lane, then the max and the row sum
    auto o_off = [&](int gi) { return ((gi * 4 + wave) * 64 + lane) * 4; };
    const int ml_off = 256 * (D / 2) + wave * 128 + lane;
    {
      const auto r = rsrc(part);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 d = {__float_as_uint(o[db][4 * i]), __float_as_uint(o[db][4 * i + 1]),
                           __float_as_uint(o[db][4 * i + 2]), __float_as_uint(o[db][4 * i + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(d, r, 4 * o_off(4 * db + i), 0, kFlashCoherent);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), r, 4 * ml_off, 0, kFlashCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lsum), r, 4 * (ml_off + 64), 0,
                                            kFlashCoherent);
    }
    // every store of the workgroup has completed before its arrival is counted
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    volatile int* last_flag = (volatile int*)Ks0;  // LDS is idle after the tile loop
    if (tid == 0) {
      int* cnt = (int*)fg.ws + split_id;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == fg.parts - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *last_flag = last;
    }
    __syncthreads();
    if (!*last_flag) return;
    // the sc1 loads see every store that completed before its piece was counted; the fence
    // keeps the compiler from hoisting them above the count. Every partial, this piece's own
    // included, is folded in piece order, so the result does not depend on which piece
    // arrived last (folding into the empty start, m = -inf, copies the first partial exactly).
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    for (int p = 0; p < fg.parts; ++p) {
      const auto r = rsrc(p);
      const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * ml_off, 0, kFlashCoherent));
      const float lp =
          __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (ml_off + 64), 0, kFlashCoherent));
      u32x4 op[4 * DB];
#pragma unroll
      for (int gi = 0; gi < 4 * DB; ++gi)
        op[gi] = __builtin_amdgcn_raw_buffer_load_b128(r, 4 * o_off(gi), 0, kFlashCoherent);
      // rescale both sides to the larger reference (an empty piece has m = -inf, l = 0, O = 0)
      const float mn = fmaxf(m, mp);
      const float base = mn == -INFINITY ? 0.f : mn;
      const float wa = fast_exp2((m - base) * c), wb = fast_exp2((mp - base) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[db][4 * i + e] = o[db][4 * i + e] * wa + __uint_as_float(op[4 * db + i][e]) * wb;
      lsum = lsum * wa + lp * wb;
      m = mn;
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  // The output goes out as whole rows. In the accumulator layout a lane holds 4 columns of
  // one query row, so a direct store instruction would touch 32 rows with 16 bytes each; each
  // wavefront instead writes its 32 x D block into one idle tile buffer (16-byte granules
  // XOR-swizzled by row) and reads it back as 16-byte granules, 4 whole rows per instruction.
  // Only this wavefront touches its buffer, and LDS operations of a wavefront complete in
  // order, so no barrier is needed between the two passes.
  constexpr int OB = D * (int)sizeof(OutT);  // bytes per output row
  constexpr int GR = OB / 16;                // 16-byte granules per row
  static_assert(32 * OB <= TILE, "a wavefront's output block must fit one tile buffer");
  if (split_id >= 0) __syncthreads();  // the merging workgroup: every wave has read last_flag
  unsigned char* const stage = wave == 0 ? Ks0 : wave == 1 ? Ks1 : wave == 2 ? Vs0 : Vs1;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int byte = (32 * db + 8 * i + 4 * hi) * (int)sizeof(OutT);
      const int pos = (((byte >> 4) ^ (l32 % GR)) << 4) | (byte & 15);
      store4<OutT>((OutT*)(stage + l32 * OB + pos), o[db][4 * i] * inv, o[db][4 * i + 1] * inv,
                   o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
    }
  // rows past Tq fall outside the store resource's range and are dropped
  const int out_stride = a.Hq * OB;           // host-checked: 32 rows of it fit an int
  const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
      (unsigned char*)a.out + (((int64_t)b * a.Tq + q0) * a.Hq + h) * OB, (short)0,
      n_qrows > 0 ? (n_qrows - 1) * out_stride + OB : 0, kBufferRsrcWord3);
  u32x4 val[GR / 2];
#pragma unroll
  for (int k = 0; k < GR / 2; ++k) {
    const int f = k * 64 + lane, row = f / GR, gr = f % GR;
    val[k] = *(const u32x4*)(stage + row * OB + ((gr ^ (row % GR)) << 4));
  }
#pragma unroll
  for (int k = 0; k < GR / 2; ++k) {
    const int f = k * 64 + lane, row = f / GR, gr = f % GR;
    __builtin_amdgcn_raw_buffer_store_b128(val[k], rout, row * out_stride + gr * 16, 0, 0);
  }
  if (q_ok && a.lse && hi == 0) {
    const float mm = m == -INFINITY ? 0.f : m;
    a.lse[((int64_t)b * a.Hq + h) * a.Tq + my_q] = mm * a.scale + logf(ltot);
  }
}

// Tail split plan. Each XCD holds kFlashSlotsPerXcd workgroups at a time; with I items per
// XCD, F = I / slots whole rounds and R = I % slots items left, the last round leaves slots
// idle. Cutting those R items into k key-range pieces makes that round ceil(R k / slots) / k
// of an item's time instead of one. k is the smallest that minimises it, and the split is
// used only if it saves at least 5% and every piece keeps kFlashMinPieceTiles tiles at the
// host's bound on the key count.
struct FlashPlan {
  int n_qtiles, nf, r, parts;
};
static FlashPlan flash_plan(int B, int Hq, int Tq, int key_bound) {
  FlashPlan pl{(Tq + kFlashBM - 1) / kFlashBM, 0, 0, 1};
  const int64_t BH = (int64_t)B * Hq;
  const int64_t items = (int64_t)pl.n_qtiles * BH;
  if (BH % 8 != 0 || items > 0x7fffffff) return pl;
  const int I = (int)(items / 8);
  pl.nf = I;
  const int F = I / kFlashSlotsPerXcd, R = I % kFlashSlotsPerXcd;
  if (F == 0 || R == 0) return pl;
  double best = F + 1.0;
  int best_k = 1;
  for (int k = 2; k <= 8; ++k) {
    if ((int64_t)key_bound < (int64_t)k * kFlashMinPieceTiles * kFlashBN) break;
    const double cost = F + (double)((R * k + kFlashSlotsPerXcd - 1) / kFlashSlotsPerXcd) / k;
    if (cost < best - 1e-9) {
      best = cost;
      best_k = k;
    }
  }
  if (best_k == 1 || best > 0.95 * (F + 1)) return pl;
  pl.nf = I - R;
  pl.r = R;
  pl.parts = best_k;
  return pl;
}

size_t flash_workspace_bytes(int B, int Hq, int Tq, int D, int key_bound) {
  const FlashPlan pl = flash_plan(B, Hq, Tq, key_bound);
  if (pl.parts == 1) return 0;
  const size_t n_split = (size_t)8 * pl.r;
  return ((size_t)flash_counter_floats((int)n_split) + n_split * pl.parts * flash_piece_floats(D)) *
         sizeof(float);
}

template <typename T, typename OutT>
static hipError_t launch_flash_t(const AttnArgs& a, int D, FlashGrid fg, hipStream_t s) {
  constexpr bool kPV16 = std::is_same<T, bf16_t>::value && std::is_same<OutT, float>::value;
  const int64_t blocks = fg.parts == 1 ? (int64_t)fg.n_qtiles * a.Hq * a.B
                                       : (int64_t)8 * (fg.nf + fg.r * fg.parts);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  if (D == 128)
    hipLaunchKernelGGL((k_attn_flash<T, 128, OutT, kPV16>), grid, block, 0, s, a, fg);
  else
    hipLaunchKernelGGL((k_attn_flash<T, 64, OutT, kPV16>), grid, block, 0, s, a, fg);
  return hipGetLastError();
}

// ws: the caller's workspace or nullptr. The tail split runs only when the plan asks for one
// and ws holds flash_workspace_bytes (16-byte aligned, counters zero); otherwise every item
// runs whole, with the same result up to the order of the final sums.
hipError_t launch_attn_flash(const AttnArgs& a, int dtype, int out_dtype, int D, int key_bound,
                             void* ws, size_t ws_bytes, hipStream_t s) {
  const FlashPlan pl = flash_plan(a.B, a.Hq, a.Tq, key_bound);
  FlashGrid fg{pl.n_qtiles, pl.nf, pl.r, pl.parts, (float*)ws};
  const size_t need = flash_workspace_bytes(a.B, a.Hq, a.Tq, D, key_bound);
  if (pl.parts == 1 || !ws || ws_bytes < need || ((uintptr_t)ws & 15)) fg = FlashGrid{pl.n_qtiles, 0, 0, 1, nullptr};
  if (dtype == SKV_BF16)
    return out_dtype == SKV_F32 ? launch_flash_t<bf16_t, float>(a, D, fg, s)
                                : launch_flash_t<bf16_t, bf16_t>(a, D, fg, s);
  return out_dtype == SKV_F32 ? launch_flash_t<f16_t, float>(a, D, fg, s)
                              : launch_flash_t<f16_t, f16_t>(a, D, fg, s);
}

}  // namespace skv
