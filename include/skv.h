/*
 * skv.h -- C ABI of libskv: KV-cache writes and chunk attention over a preallocated
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (web pages; cited by title and section):
 *   [LB]  LingBot-World PR #53 "refactor(kv): index_copy_ for KV-cache writes (enabler for
 *         multi-user batching + CUDA Graphs)"
 *   [FD]  flashdreams issue #763 "add an opt-in circular KV policy for streaming attention"
 *   [FS]  fish-speech PR #1312 "perf(text2semantic): pass only active KV cache prefix to SDPA"
 *   [TR]  TensorRT-LLM PR #18973 "FA4 variable-length cross-attention"
 *
 * Conventions shared by every entry point
 *   - Returns an skv_status; never throws, never synchronizes the device, never allocates
 *     device memory (all device buffers, including ring metadata and attention workspace,
 *     are owned by the caller), never reads device memory on the host. Work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream). Together these make
 *     every call safe to record into a HIP graph: changing positions, slots and lengths live
 *     in device memory the kernels read at run time [FD, proposed boundary: captured kernels
 *     must take the changing slot from device data].
 *   - A non-OK status means nothing was enqueued; skv_last_error() then returns a message
 *     (thread-local, valid until the next call on the same thread).
 *   - Optional arguments are NULL / 0 and then fall back to the plain path, as the new
 *     keyword arguments of [LB, Non-regressive design] default to None.
 *   - Tensors are dense, row-major, with the shapes given per call; device pointers must be
 *     16-byte aligned (SKV_ERR_ALIGN otherwise).
 *   - Errors only the device can see (an index out of range, a device kv_len outside
 *     [1, cap], a bad cu_seqlens_kv segment, a ring write with no reservation) OR a bit
 *     (SKV_DEV_*) into *err_dev when err_dev is non-NULL; the offending rows / batch
 *     elements are skipped (their outputs are unspecified) and no memory outside the
 *     arguments is touched. The caller clears *err_dev.
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_ERR_NULL = 1,        /* a required pointer is NULL */
  SKV_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. Hq not a multiple of Hkv) */
  SKV_ERR_RANGE = 3,       /* a host-side value outside its valid range (e.g. kv_len) */
  SKV_ERR_DTYPE = 4,       /* unknown dtype or unsupported dtype combination */
  SKV_ERR_ALIGN = 5,       /* a device pointer or row size not 16-byte aligned */
  SKV_ERR_UNSUPPORTED = 6, /* a valid request this library does not implement (e.g. D=96,
                              packed K/V with the full-capacity arm) [TR, Acceptance
                              criteria: explicit capability check instead of a silent path] */
  SKV_ERR_HIP = 7          /* the HIP runtime refused a launch */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_F16 = 1, SKV_BF16 = 2 } skv_dtype;

/* Bits OR-ed into *err_dev by kernels. */
enum {
  SKV_DEV_INDEX_RANGE = 1,   /* a write index outside [0, cap): that row was not written */
  SKV_DEV_KV_LEN = 2,        /* a device kv_len outside [1, cap] or shorter than a causal
                                chunk: that batch element was skipped */
  SKV_DEV_CU_SEQLENS = 4,    /* cu_seqlens_kv not starting at 0, not increasing, or a
                                zero-length segment: that batch element was skipped */
  SKV_DEV_RING_UNRESERVED = 8, /* ring write for a batch element with no reserved slot */
  SKV_DEV_CURSOR_FULL = 16   /* cursor advance past the capacity: cursor left unchanged */
};

const char* skv_last_error(void);
const char* skv_version(void);

/* ------------------------------------------------------------------------------------
 * Indexed slab write [LB, Summary; What this is and isn't]
 *
 * index_copy along the sequence dimension, for K and V in one launch:
 *     k_cache[b, index[t], :, :] = k_src[b, t, :, :]   (and the same for V)
 * for b < B, t < n. k_cache/v_cache: [B, cap, Hkv, D]; k_src/v_src: [B, n, Hkv, D]; all of
 * `dtype`. index_dev: int64 [n] on the device, one vector shared by every batch element
 * (homogeneous multi-user batching). index_dev == NULL writes the contiguous rows
 * [start, start+n) -- the slice assignment cache[:, start:start+n] = src -- and the host
 * checks that range (SKV_ERR_RANGE). v_cache and v_src may both be NULL (K only).
 * Indices are expected unique (duplicates leave an unspecified one of the rows); an index
 * outside [0, cap) skips that row and sets SKV_DEV_INDEX_RANGE. n == 0 or B == 0: no-op.
 * ------------------------------------------------------------------------------------ */
skv_status kv_write_indexed(void* k_cache, void* v_cache, const void* k_src, const void* v_src,
                            const int64_t* index_dev, int64_t start, int B, int cap, int n,
                            int Hkv, int D, int dtype, int32_t* err_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * Writes with keys rotated at their absolute positions [FD, proposed boundary: keys whose
 * rotary embedding is applied before the cache write, at absolute positions]
 *
 * The page gives no formula; these entry points implement 1-D rotary embedding. For each key
 * row (every head) and pair index i < D/2, the coordinates (a, b) of pair i -- (i, i + D/2)
 * for SKV_ROPE_HALF, (2i, 2i + 1) for SKV_ROPE_INTERLEAVED -- become
 *     (a cos(theta) - b sin(theta), a sin(theta) + b cos(theta)),  theta = pos * inv_freq[i],
 * computed in fp64 (no fused multiply-add), rounded to fp32 and then to the cache dtype
 * (round to nearest even). inv_freq_dev: double [D/2] on the device, 8-byte aligned, the
 * caller's frequencies (e.g. base^(-2i/D)). V rows are stored unchanged. D must be a power of
 * two in [16, 4096] (else SKV_ERR_SHAPE); other errors as for the plain writes.
 *
 * kv_write_indexed_rope: kv_write_indexed with K rotated at pos = its destination row
 *     (index_dev[t], or start + t when index_dev is NULL).
 * kv_ring_write_rope: kv_ring_write with K rotated at pos = chunk_id * chunk + t, where
 *     chunk_id counts the chunks reserved before the current one since the last reset (the
 *     sink chunk is 0), read from the ring's device metadata -- so the repeated denoising
 *     writes of one chunk rotate identically, and the positions follow time, not slots.
 * ------------------------------------------------------------------------------------ */
typedef enum { SKV_ROPE_HALF = 0, SKV_ROPE_INTERLEAVED = 1 } skv_rope_layout;

skv_status kv_write_indexed_rope(void* k_cache, void* v_cache, const void* k_src,
                                 const void* v_src, const int64_t* index_dev, int64_t start, int B,
                                 int cap, int n, int Hkv, int D, int dtype,
                                 const double* inv_freq_dev, int rope_layout, int32_t* err_dev,
                                 void* stream);

/* ------------------------------------------------------------------------------------
 * Device write cursor [LB, What this is and isn't: the write offset and the read slice must
 * stop being host integers for graph capture; FD, proposed boundary]
 *
 * One launch: c = *cursor_dev; if c + n <= cap:
 *     index_out_dev[t] = c + t (t < n, int64), kv_len_out_dev[b] = c + n (b < B, int32),
 *     *cursor_dev = c + n;
 * else index_out_dev[t] = -1 (so a following write skips every row), kv_len_out_dev is left
 * unchanged, the cursor is unchanged and SKV_DEV_CURSOR_FULL is set. kv_len_out_dev may be
 * NULL. The index feeds kv_write_indexed, kv_len_out feeds attn_chunk_fwd's kv_len_dev.
 * ------------------------------------------------------------------------------------ */
skv_status kv_cursor_advance(int32_t* cursor_dev, int n, int cap, int B, int64_t* index_out_dev,
                             int32_t* kv_len_out_dev, int32_t* err_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * Sink-plus-window ring [FD, current path; proposed boundary; first experiment]
 *
 * Storage k_store/v_store: [B, n_slots*chunk, Hkv, D] (caller-owned, stable). Each batch
 * element (e.g. the cond and uncond CFG branches) has independent state in meta_dev
 * (kv_ring_meta_bytes(B) bytes of caller device memory, 4-byte aligned):
 *     counter[b]  chunks reserved since reset      slot[b]   slot of the current chunk or -1
 *     pending[b]  reserved but not yet written      valid[b]  tokens attention may read
 * Slots: the first sink_slots chunks since reset stay pinned; after the storage fills, a new
 * chunk replaces the oldest non-sink chunk: chunk c goes to slot c while c < n_slots, else
 * to sink + (c - sink) mod (n_slots - sink). The occupied slots are therefore always the
 * physical prefix [0, valid/chunk), and because unmasked attention does not depend on the
 * order of (key, value) rows [FD, proposed boundary], attention reads the ring through
 * kv_ring_kv_len_dev() as an active prefix with no gather.
 *
 * Reservation is separate from writes [FD, proposed boundary]: kv_ring_reserve picks the
 * slot of the next chunk (a reserve while the previous reservation is still unwritten keeps
 * it); every kv_ring_write then overwrites that slot (the repeated denoising writes of one
 * chunk); the first write after a reserve commits valid[b] = min(counter, n_slots)*chunk.
 * kv_ring_reset forgets the contents (counter 0, slot -1, valid 0) without touching storage.
 * batch_mask_dev: uint8 [B] on the device, nonzero = act on that element; NULL = all.
 * The handle is a small host-side descriptor (malloc'd by create, freed by destroy); it
 * holds the pointers and sizes given to create.
 * ------------------------------------------------------------------------------------ */
typedef struct skv_ring skv_ring;

size_t kv_ring_meta_bytes(int B);
/* Enqueues the metadata initialisation (a kernel, no memset) on `stream`.
   Requires 0 <= sink_slots < n_slots, chunk >= 1. */
skv_status kv_ring_create(skv_ring** out, void* k_store, void* v_store, void* meta_dev, int B,
                          int chunk, int n_slots, int sink_slots, int Hkv, int D, int dtype,
                          void* stream);
skv_status kv_ring_reserve(skv_ring* ring, const uint8_t* batch_mask_dev, void* stream);
/* k_src/v_src: [B, chunk, Hkv, D]; v_src NULL iff the ring has no V storage. */
skv_status kv_ring_write(skv_ring* ring, const void* k_src, const void* v_src,
                         const uint8_t* batch_mask_dev, int32_t* err_dev, void* stream);
/* kv_ring_write with keys rotated at their chronological positions (see the section on
   rotary writes above). */
skv_status kv_ring_write_rope(skv_ring* ring, const void* k_src, const void* v_src,
                              const double* inv_freq_dev, int rope_layout,
                              const uint8_t* batch_mask_dev, int32_t* err_dev, void* stream);
skv_status kv_ring_reset(skv_ring* ring, const uint8_t* batch_mask_dev, void* stream);
const int32_t* kv_ring_kv_len_dev(const skv_ring* ring); /* valid[B], device */
const int32_t* kv_ring_slot_dev(const skv_ring* ring);   /* slot[B], device */
skv_status kv_ring_destroy(skv_ring* ring);

/* ------------------------------------------------------------------------------------
 * Roll-left of a chronological window: the comparison arm [FD, current path]
 *
 * The cache the ring replaces keeps rows in time order, sink first; when a new chunk
 * overflows the window, the retained non-sink rows move left by one chunk, and the new chunk
 * is then written at the end (kv_write_indexed at rows [rows - shift_rows, rows)).
 * kv_roll_left moves rows [sink_rows + shift_rows, rows) of every batch element of
 * k_store / v_store [B, rows, Hkv, D] to [sink_rows, rows - shift_rows), with memmove
 * semantics (source and destination overlap): it enqueues copies of at most shift_rows rows
 * in increasing row order on `stream`, each reading rows that no earlier copy writes. Rows
 * [rows - shift_rows, rows) keep their old contents. v_store NULL: K only. Requires
 * 0 <= sink_rows, 1 <= shift_rows, sink_rows + shift_rows <= rows (equality: nothing moves).
 * ------------------------------------------------------------------------------------ */
skv_status kv_roll_left(void* k_store, void* v_store, int B, int rows, int sink_rows,
                        int shift_rows, int Hkv, int D, int dtype, void* stream);

/* ------------------------------------------------------------------------------------
 * Ragged K/V packing [TR, Description; Acceptance criteria]
 *
 * kv_ragged_metadata: cu_seqlens_out_dev[0] = 0 and cu[b+1] = cu[b] + lens_dev[b] (int32
 * [B] in, int32 [B+1] out, device, one launch). A length outside [0, max_kv] counts as 0 and
 * sets SKV_DEV_KV_LEN. The metadata depends only on the length layout, so it is prepared once
 * per layout [TR, Description]; attention then takes cu_seqlens_kv with max_seqlen_kv = max_kv.
 * kv_pack_ragged: for every b, rows [0, len_b) of k_padded / v_padded [B, max_kv, Hkv, D] go
 * to rows [cu[b], cu[b] + len_b) of k_packed / v_packed [packed_rows, Hkv, D], where
 * len_b = cu[b+1] - cu[b] (the key padding is at the end of each branch). A segment that
 * does not fit (cu[b] < 0, len_b < 0 or > max_kv, cu[b+1] > packed_rows) is skipped and sets
 * SKV_DEV_CU_SEQLENS. v_packed / v_padded NULL: K only. With packed_rows == 0 the packed
 * pointers may be NULL: no row is written, and any non-empty segment sets SKV_DEV_CU_SEQLENS.
 * ------------------------------------------------------------------------------------ */
skv_status kv_ragged_metadata(const int32_t* lens_dev, int B, int max_kv, int32_t* cu_seqlens_out_dev,
                              int32_t* err_dev, void* stream);
skv_status kv_pack_ragged(void* k_packed, void* v_packed, const void* k_padded, const void* v_padded,
                          const int32_t* cu_seqlens_dev, int B, int max_kv, int packed_rows, int Hkv,
                          int D, int dtype, int32_t* err_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * Chunk attention over a KV cache [FS, Problem; Change] [TR, Description]
 *
 *     out[b, t, h, :] = sum_j softmax_j(scale * <q[b,t,h,:], k_j>) v_j
 * over the key set J(b, t):
 *   prefix mode   (cu_seqlens_kv_dev == NULL): keys are rows [0, kv_len_b) of
 *                 k/v [B, cap, Hkv, D], kv_len_b = kv_len_dev[b] if kv_len_dev else kv_len;
 *                 1 <= kv_len_b <= cap [FS, author's reply: 1 and cap valid, 0 and cap+1 not].
 *   packed mode   (cu_seqlens_kv_dev != NULL): keys of b are rows [cu[b], cu[b+1]) of
 *                 k/v [cap, Hkv, D] (cap = rows allocated in the packed buffer; a segment
 *                 ending past it is a device error); q stays padded [TR, Description]. cu
 *                 is int32 [B+1] on the device, prepared once by the caller and reused
 *                 [TR, Description].
 *   SKV_FULL_CAPACITY_MASKED (prefix mode only): the comparison arm -- every one of the cap
 *                 rows is visited and rows j >= kv_len_b are masked out [FS, Problem].
 * Masks, with queries bottom-right aligned (query t at position p = kv_len_b - Tq + t;
 * the causal mask is cut to the active key length [FS, Change]):
 *   SKV_MASK_NONE, SKV_MASK_CAUSAL (j <= p), SKV_MASK_BLOCK_CAUSAL (j/mask_block <=
 *   p/mask_block, integer division; mask_block = 1 is CAUSAL).
 * GQA: query head h reads KV head h / (Hq/Hkv); heads are never expanded [FS, Problem].
 * q, out: [B, Tq, Hq, D]; lse (optional, fp32 [B, Hq, Tq]) = natural-log sum of
 * exp(scale*score). scale == 0 means 1/sqrt(D). D in {64, 128}; B*Tq*Hq < 2^31 and
 * Hq*D <= 2^21 (else SKV_ERR_SHAPE).
 * dtype: SKV_F32 (exact fp32 arithmetic), SKV_BF16 or SKV_F16 (matrix-core products with
 * fp32 accumulation and fp32 softmax). out_dtype: dtype or SKV_F32.
 * Workspace (caller device memory, 16-byte aligned, attn_workspace_bytes(params) bytes):
 *   - Tq <= 4 (decode-sized chunks) in bf16/f16 uses a split-K path that requires it;
 *   - larger bf16/f16 chunks take it optionally: when attn_workspace_bytes() is nonzero for
 *     them, the last, partly filled round of workgroups would leave CU slots idle, and a
 *     workspace of that size lets the kernel cut that round's items into key-range pieces
 *     merged in the same launch. Without one (NULL or smaller) every item runs whole; the
 *     results agree up to the order of the final sums;
 *   - fp32 needs none.
 * The workspace must be zero-filled once before its first use: its first 64 KiB hold arrival
 * counters (int32) that every call leaves at zero again, and every kind of call keeps its
 * partial results after those 64 KiB, so one zero-filled workspace of the largest size needed
 * can serve any later sequence of calls. Calls sharing one workspace must not overlap in time
 * (they are ordered when issued on one stream). Decode-sized chunks take the split-K path only
 * while B*Hkv < 16384 (one counter per batch element and KV head); larger batches of them
 * run the chunk path (attn_decode_step returns SKV_ERR_UNSUPPORTED).
 * max_seqlen_kv: optional host bound on any batch element's key count; it only sizes the
 * split grids and the workspace when the lengths live on the device (0 = use cap / the host
 * kv_len).
 * ------------------------------------------------------------------------------------ */
typedef enum {
  SKV_MASK_NONE = 0,
  SKV_MASK_CAUSAL = 1,
  SKV_MASK_BLOCK_CAUSAL = 2
} skv_mask;

enum { SKV_FULL_CAPACITY_MASKED = 1u };

typedef struct {
  int B, Tq, Hq, Hkv, D;
  int dtype;                        /* skv_dtype of q, k, v */
  int out_dtype;                    /* skv_dtype of out: dtype or SKV_F32 */
  int cap;                          /* rows per batch element of k/v (prefix mode), or
                                       rows of the packed k/v buffer (packed mode) */
  int kv_len;                       /* host active prefix, used iff kv_len_dev == NULL */
  const int32_t* kv_len_dev;        /* [B] device active prefixes (ring, cursor, graphs) */
  const int32_t* cu_seqlens_kv_dev; /* [B+1] device; non-NULL selects packed mode */
  int max_seqlen_kv;                /* optional host bound, see above */
  int mask;                         /* skv_mask */
  int mask_block;                   /* block size for SKV_MASK_BLOCK_CAUSAL (>= 1) */
  float scale;                      /* 0 => 1/sqrt(D) */
  unsigned flags;                   /* SKV_FULL_CAPACITY_MASKED */
  void* workspace;                  /* device, >= attn_workspace_bytes() */
  size_t workspace_bytes;
  int32_t* err_dev;                 /* optional device error word */
} skv_attn_params;

/* Bytes of workspace a call with these parameters needs (0: none); (size_t)-1 when the
   parameters are invalid (the status attn_chunk_fwd would return is then described by
   skv_last_error()). */
size_t attn_workspace_bytes(const skv_attn_params* params);
skv_status attn_chunk_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          const skv_attn_params* params, void* stream);

/* ------------------------------------------------------------------------------------
 * Fused decode step [FS, Change: decode step i writes position T+i and attends over
 * kv_len = T+i+1] [LB, What this is and isn't; FD, proposed boundary: positions on the device]
 *
 * One launch with the effect of kv_cursor_advance(cursor_dev, Tq, cap, ...) +
 * kv_write_indexed(k_cache, v_cache, k_new, v_new, index) + attn_chunk_fwd(q, k_cache, v_cache,
 * kv_len_dev = the advanced lengths): c = *cursor_dev; for every batch element b the new rows
 * k_new/v_new [B, Tq, Hkv, D] are stored at cache rows c .. c+Tq-1 of k_cache/v_cache
 * [B, cap, Hkv, D]; out = attention of q [B, Tq, Hq, D] over rows [0, c+Tq) (params->mask
 * applies, queries bottom-right aligned); then *cursor_dev = c+Tq and, if non-NULL,
 * kv_len_out_dev[b] = c+Tq. If c+Tq > cap nothing is written, the cursor stays, outputs are
 * zero and SKV_DEV_CURSOR_FULL is set. Outputs equal the three-call sequence bit for bit.
 * params: prefix mode with kv_len_dev = cu_seqlens_kv_dev = NULL and no full-capacity flag
 * (SKV_ERR_UNSUPPORTED otherwise); params->kv_len is ignored; bf16/f16 with Tq <= 4 and
 * Tq*Hq/Hkv <= 16. The workspace follows attn_workspace_bytes() of the same params (zero-filled
 * before first use, left zero-filled); max_seqlen_kv bounds c+Tq for grid sizing (0 = cap).
 * ------------------------------------------------------------------------------------ */
skv_status attn_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                            void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                            int32_t* kv_len_out_dev, const skv_attn_params* params, void* stream);

/* ------------------------------------------------------------------------------------
 * Fused decode step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): attn_decode_step with the
 * split-K scratch (arrival counters and partials) in a static array the library holds on each
 * GPU it runs on, SKV_DECODE_STATIC_SCRATCH_BYTES per GPU, kept until the process ends.
 *
 * Arguments, results and device errors are those of attn_decode_step; params->workspace and
 * params->workspace_bytes are ignored. A step whose scratch need (attn_workspace_bytes() of
 * the same parameters; it grows with B*Hkv and the key bound) exceeds
 * SKV_DECODE_STATIC_SCRATCH_BYTES returns SKV_ERR_RANGE and launches nothing. The call
 * allocates nothing; its first call on a GPU looks up that GPU's array (that device must be
 * current) and clears its counters with a kernel on `stream`, and every call leaves them
 * cleared. All calls on one GPU share its array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and give undefined
 * results; calls issued on one stream are ordered.
 * ------------------------------------------------------------------------------------ */
#define SKV_DECODE_STATIC_SCRATCH_BYTES (4u << 20)
skv_status attn_decode_step_static(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, void* out, float* lse, int32_t* cursor_dev,
                                   int32_t* kv_len_out_dev, const skv_attn_params* params,
                                   void* stream);

/* ------------------------------------------------------------------------------------
 * Measurement probes (not part of the hot path): ceilings measured on the chip by kernels of
 * this library, against which the hot-path kernels are also reported (the nominal peaks of
 * the data sheet assume a 2.4 GHz clock the chip does not hold under matrix-core load).
 *
 * skv_probe_mfma_bf16: `workgroups` workgroups of 4 wavefronts, each wavefront issuing
 *   4 * iters v_mfma_f32_32x32x16_bf16 from registers (32768 flops each, so
 *   workgroups * 16 * iters * 32768 flops in all), then writing one float per lane to out_dev
 *   [workgroups * 256] (caller device memory; the values are meaningless).
 * skv_probe_copy: copies `bytes` (a multiple of 16) from src_dev to dst_dev (device, 16-byte
 *   aligned, not overlapping) with the cache writes' access pattern; 2 * bytes of traffic.
 * Errors: SKV_ERR_NULL, SKV_ERR_RANGE / SKV_ERR_SHAPE for sizes, SKV_ERR_ALIGN.
 * ------------------------------------------------------------------------------------ */
skv_status skv_probe_mfma_bf16(float* out_dev, int workgroups, int iters, void* stream);
skv_status skv_probe_copy(void* dst_dev, const void* src_dev, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SKV_H */
