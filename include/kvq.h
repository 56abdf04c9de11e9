/*
 * kvq.h — C ABI of libkvq: an INT8-quantized KV cache for AMD MI355X (gfx950).
 *
 * What the library computes (sources are docs.rs source pages, cited by page
 * title and Rust item):
 *   - quantize-on-append: symmetric absmax/127 codes stored as u8 with a +128
 *     offset, one fp32 scale per token row or per 32 elements along head_dim
 *     (abaddon 0.2.0-rc.1 src/kv_cache_quant_cuda.rs, `quantize_tensor`;
 *     combs-models 0.2.2 src/kv.rs, `kv_quantize`; realizar 0.8.5
 *     src/cuda/executor/kv_cache_q8_init.rs, `init_kv_cache_q8_gpu`);
 *   - attention directly on those codes, dequantizing in registers
 *     (abaddon kv_cache_quant_cuda.rs module doc, "fused approach"), over GQA
 *     heads, in a contiguous or a paged (16-token pages) layout (combs-models
 *     kv.rs, `PagedKVCache`, `attend`).
 *
 * Conventions (every entry point):
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no global mutable state besides a thread-local
 *     error message, never synchronizes and never reads device memory on the
 *     host.  Work is enqueued on `stream` (a hipStream_t; NULL = null stream).
 *   - Return value: KVQ_OK, or an error code with a message available from
 *     kvq_last_error() on the calling thread.  On error nothing is enqueued.
 *   - Layouts (row-major, last index fastest):
 *       new K/V rows       [batch, num_kv_heads, n_new, head_dim]
 *       queries / outputs  [batch, num_heads, n, head_dim]   (n = 1: [B, H, D])
 *       contiguous cache   codes [batch, num_kv_heads, max_len, head_dim] u8,
 *                          scales [batch, num_kv_heads, max_len, G] fp32
 *       paged arena        codes [num_pages, num_kv_heads, 16, head_dim] u8,
 *                          scales [num_pages, num_kv_heads, 16, G] fp32,
 *                          block_table [batch, max_blocks_per_seq] int32
 *     with G = 1 (KVQ_SCALE_PER_TOKEN) or head_dim/32 (KVQ_SCALE_GROUP32).
 *   - GQA: query head h reads KV head h / (num_heads / num_kv_heads)
 *     (combs-models kv.rs, `repeat_kv`).
 *   - Host-checkable argument errors return KVQ_ERR_INVALID_ARG (null
 *     pointer, num_heads % num_kv_heads != 0, head_dim not a multiple of 32 or
 *     above 256, paged page_size != 16, n_new <= 0, ...).  Device-side values
 *     (positions, lengths, page ids) are the caller's contract; kernels clamp
 *     or skip out-of-range ones so that no access leaves the buffers described
 *     by the descriptor.  A library built with -DKVQ_DEBUG (build.py --debug,
 *     int8_quantized_kv_amd/_dbg/libkvq.so) checks them on the host before
 *     each attention launch: it waits for the stream, copies the lengths and
 *     the block table, and returns KVQ_ERR_OUT_OF_RANGE, launching nothing,
 *     when a length passes its bound or a page the call reads lies outside
 *     [0, num_pages).  For testing; the release build never reads device
 *     memory on the host.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1,  /* bad descriptor or argument (host-checkable)        */
  KVQ_ERR_OUT_OF_RANGE = 2, /* host-known size beyond the cache capacity          */
  KVQ_ERR_UNSUPPORTED = 3,  /* valid but not implemented (e.g. FP8 recent window) */
  KVQ_ERR_HIP = 4,          /* kernel launch failed (hipGetLastError)             */
  KVQ_ERR_WORKSPACE = 5     /* workspace missing or smaller than required          */
} kvq_status;

/* Scale modes.  KVQ_SCALE_PER_TOKEN_BF16 (abaddon kv_cache_quant_cuda.rs,
 * `CudaQuantizedKvCache::quantize_tensor`): the codes come from the fp32
 * per-token scale exactly as in KVQ_SCALE_PER_TOKEN, and the scale is stored
 * rounded to bf16 (nearest even), which every reader then multiplies by (the
 * page's own mismatch: the dequantization error can exceed half a step).  In
 * that mode k_scales / v_scales point to uint16 bf16 arrays of the same
 * shape (4-byte aligned, as every scale array must be: kernels read the
 * aligned word holding a scale).  Every entry point accepts this mode.
 *
 * FP8 code formats (llama-gguf 0.14.0 src/model/kv_quantized.rs,
 * `KVCacheFormat::Fp8E4M3` / `Fp8E5M2`), set in the same field: each element
 * is stored as one FP8 byte of its own value, with no scale (k_scales /
 * v_scales are unused and may be NULL).  The encoder is the page's
 * `quantize_fp8_e4m3` / `quantize_fp8_e5m2`: the value is cut toward zero
 * onto the format's grid; E4M3 inputs of magnitude 512 and above saturate to
 * +/-448 and E5M2 inputs of 131072 and above to +/-inf; below that, the top
 * exponent field is kept, so E4M3 magnitudes in [480, 512) take the NaN code
 * and E5M2 magnitudes in [65536, 131072) the inf and NaN codes, as on the
 * page.  Readers decode as the page's `dequantize_fp8_*` (the OCP values;
 * negative zero reads as +0).  Attention over a non-finite code is
 * non-finite.  Decode attention, chunked attention and dequantization
 * support both formats; a recent window over FP8 codes returns
 * KVQ_ERR_UNSUPPORTED.
 *
 * Block scales (abaddon kv_cache_quant_cuda.rs, `QuantGranularity::PerHead` /
 * `PerChannel`, `quantize_with_granularity`), for hybrid caches only: the
 * page's per-head scale (maximum over the sequence and head_dim) and
 * per-channel scale (maximum over the sequence, one per element index) are
 * taken over fixed, position-aligned blocks of 16 rows of one (sequence, KV
 * head), so that the codes depend on the token history alone.  Block j
 * (positions 16j .. 16j+15) is quantized from its rows' bf16 values when its
 * first row leaves the recent window; the window must be at least 15 so that
 * all 16 rows exist then.  Positions below L - window read as INT8, as in the
 * per-token hybrid cache.
 *   KVQ_SCALE_BLOCK_HEAD    : one scale per (block, KV head), stored once
 *                             per row, like per-token scales (G = 1), so the
 *                             per-token kernels read it unchanged.
 *   KVQ_SCALE_BLOCK_CHANNEL : head_dim scales per (block, KV head): contiguous
 *                             [batch, num_kv_heads, max_len/16, head_dim],
 *                             paged [num_pages, num_kv_heads, head_dim] (a
 *                             page is one block).
 * Contiguous caches in these modes need max_len % 16 == 0.  Only the
 * recent-window entry points (kvq_*_recent) take them; the others return
 * KVQ_ERR_UNSUPPORTED. */
enum {
  KVQ_SCALE_PER_TOKEN = 0,
  KVQ_SCALE_GROUP32 = 1,
  KVQ_SCALE_PER_TOKEN_BF16 = 2,
  KVQ_CODES_FP8_E4M3 = 3,
  KVQ_CODES_FP8_E5M2 = 4,
  KVQ_SCALE_BLOCK_HEAD = 5,
  KVQ_SCALE_BLOCK_CHANNEL = 6
};
enum { KVQ_LAYOUT_CONTIGUOUS = 0, KVQ_LAYOUT_PAGED = 1 };
enum { KVQ_DT_F32 = 0, KVQ_DT_BF16 = 1 };

/* One layer's K/V cache (the pages keep one cache per layer: realizar
 * kv_cache_q8_init.rs per-layer buffers; combs-models kv.rs per-layer arena). */
typedef struct kvq_cache {
  int32_t batch;               /* sequences                                       */
  int32_t num_heads;           /* query heads H                                   */
  int32_t num_kv_heads;        /* KV heads KVH, H % KVH == 0                      */
  int32_t head_dim;            /* D: multiple of 32, at most 256                  */
  int32_t layout;              /* KVQ_LAYOUT_*                                    */
  int32_t scale_mode;          /* KVQ_SCALE_* (INT8 codes) or KVQ_CODES_FP8_*     */
  int32_t max_len;             /* contiguous: per-sequence capacity (tokens)      */
  int32_t page_size;           /* paged: must be 16                               */
  int32_t num_pages;           /* paged: arena pages P                            */
  int32_t max_blocks_per_seq;  /* paged: block-table row length                   */
  const int32_t* block_table;  /* paged: device [batch, max_blocks_per_seq]       */
  uint8_t* k_codes;            /* device, layout above                            */
  uint8_t* v_codes;
  float* k_scales;             /* fp32 (bf16 in KVQ_SCALE_PER_TOKEN_BF16; unused
                                  for FP8 codes)                                  */
  float* v_scales;
} kvq_cache;

/*
 * kvq_append — quantize n_new new K and V rows per (sequence, KV head) and
 * write them at logical positions start_pos[b] .. start_pos[b] + n_new - 1.
 *
 * Follows abaddon kv_cache_quant_cuda.rs `CudaQuantizedKvCache::quantize_tensor`
 * step by step in IEEE fp32: m = max(max|x|, 1e-8); s = m / 127 (correctly
 * rounded); q = round-half-away-from-zero(x / s) (correctly rounded quotient);
 * code = q + 128 in [1, 255].  Group-32 scales take the max over 32 elements
 * (combs-models kv.rs `kv_quantize`); scales are stored as fp32 (realizar
 * kv_cache_q8_init.rs).  The slot write is a fixed-capacity store: contiguous
 * row (b, h, p) sits at ((b*KVH + h)*max_len + p); paged position p of
 * sequence b sits in page block_table[b][p/16], slot p%16 (combs-models kv.rs
 * `PagedKVCache::attention_opts` write loop).  FP8 code formats store
 * each element's own byte from the page's encoder instead (see the scale
 * modes above) and write no scales.
 *
 *   k_new, v_new : device [B, KVH, n_new, D], fp32 or bf16 (in_dtype)
 *   start_pos    : device int32 [B]
 * Errors: INVALID_ARG (nulls, bad descriptor, n_new <= 0, bad dtype),
 * OUT_OF_RANGE (n_new larger than the per-sequence capacity).  Rows whose
 * device position or page id falls outside the cache are not written.
 */
kvq_status kvq_append(const kvq_cache* cache, const void* k_new, const void* v_new,
                      int32_t in_dtype, int32_t n_new, const int32_t* start_pos,
                      void* stream);

/*
 * kvq_attention_decode — one query token per sequence attends to the first
 * seq_lens[b] cached tokens (the tokens appended for this step included; a
 * decode query at the end of the window needs no mask: combs-models kv.rs
 * `attend`).  out[b,h,:] = softmax_t(attn_scale * q.k_hat_t) . v_hat_t with
 * k_hat = (code - 128) * scale dequantized in registers (abaddon
 * kv_cache_quant_cuda.rs module doc, fused approach), or the decoded value
 * of an FP8 code.  Computed as split-K
 * partials (m, l, o) per token range, merged with a log-sum-exp combine; the
 * result is rounded to bf16 (nearest even).
 *
 *   q         : device bf16 [B, H, D]
 *   seq_lens  : device int32 [B]; each in [1, max_seq_len_hint] (values are
 *               clamped to [0, min(hint, capacity)]; a length of 0 gives zeros)
 *   out       : device bf16 [B, H, D]
 *   workspace : device scratch of at least kvq_workspace_size(cache,
 *               max_seq_len_hint, 1) bytes: split merge counters, then
 *               split partials (a partial word reads zero until its split
 *               has written it).  Zero-fill it once after allocation; every
 *               call of this library returns the whole workspace to zero,
 *               so it can be reused by later calls on the same stream, of
 *               any entry point.  Calls that overlap in time (other streams)
 *               must not share a workspace.
 * Errors: INVALID_ARG, OUT_OF_RANGE (hint beyond capacity or < 1),
 * WORKSPACE, HIP.  Head dims 32, 64 and 128 run on the streaming kernel; the
 * other multiples of 32 up to 256 on a generic kernel (fp32 arithmetic,
 * a separate merge launch).
 */
kvq_status kvq_attention_decode(const kvq_cache* cache, const uint16_t* q,
                                const int32_t* seq_lens, float attn_scale, uint16_t* out,
                                void* workspace, size_t workspace_bytes,
                                int32_t max_seq_len_hint, void* stream);

/*
 * kvq_append_decode — one decode step in a single launch: the new K and V
 * rows of every sequence are quantized into position seq_lens[b] - 1 (exactly
 * as kvq_append with start_pos = seq_lens - 1 and n_new = 1 would), then the
 * query attends to the first seq_lens[b] tokens, that row included (exactly
 * as kvq_attention_decode).  The workgroup whose token range holds the new
 * position quantizes the rows and uses them directly, so no separate append
 * pass runs first.
 *
 *   k_new, v_new : device [B, KVH, 1, D] of in_dtype (fp32 or bf16)
 *   other arguments and the workspace as for kvq_attention_decode; a
 *   sequence with seq_lens[b] <= 0 writes no row and gives zeros.
 * Errors: those of kvq_append and kvq_attention_decode.
 */
kvq_status kvq_append_decode(const kvq_cache* cache, const void* k_new, const void* v_new,
                             int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens,
                             float attn_scale, uint16_t* out, void* workspace,
                             size_t workspace_bytes, int32_t max_seq_len_hint, void* stream);

/*
 * kvq_attention_chunk — chunked prefill: n queries per sequence, already
 * appended at positions ctx_lens[b] .. ctx_lens[b] + n - 1, attend to the
 * cache.  With causal != 0 query i sees keys t <= ctx_lens[b] + i
 * (bottom-right alignment: abaddon kv_cache_quant_cuda.rs
 * `forward_attention`, cache_offset = seq_len - q_len; combs-models kv.rs
 * `attend`); otherwise all ctx_lens[b] + n keys.  Both products run on
 * f16 MFMA with the codes as exact f16 values and the scales applied to the
 * fp32 scores and weights (group-32 K scales to the fp32 score accumulator
 * group by group; group-32 V ratios to the f16 weights of each 32-dim output
 * tile); bf16 output.  Head dims other than 64 and 128 run instead as one
 * decode per (sequence, query) over the keys that query sees (fp32
 * arithmetic, split partials in the workspace; batch * n at most 65535).
 *
 *   q        : device bf16 [B, H, n, D];  out : device bf16 [B, H, n, D]
 *   ctx_lens : device int32 [B], tokens cached before the chunk
 *   max_ctx_len_hint : host upper bound on ctx_lens; hint + n must fit the
 *              capacity
 *   workspace: kvq_workspace_size(cache, max_ctx_len_hint + n, n) bytes
 *              (kvq_workspace_size_window with the window): 0 for head dims
 *              64 and 128, where NULL is accepted
 * Keys beyond the cache capacity do not exist: a query sees at most
 * min(ctx_lens[b] + n, capacity) keys.
 * Errors: INVALID_ARG, OUT_OF_RANGE (batch * n above 65535 for head dims
 * other than 64 and 128), WORKSPACE, HIP.
 */
kvq_status kvq_attention_chunk(const kvq_cache* cache, const uint16_t* q, int32_t n,
                               const int32_t* ctx_lens, int32_t causal, float attn_scale,
                               uint16_t* out, void* workspace, size_t workspace_bytes,
                               int32_t max_ctx_len_hint, void* stream);

/*
 * kvq_dequant — materialise one cache side as values: out[b,h,t,d] =
 * fl32((code - 128) * scale) (abaddon kv_cache_quant_cuda.rs
 * `int8_dequant_bf16`; abaddon 0.2.0-rc.2 kv_cache_quant.rs `dequantize`),
 * or an FP8 code's value as the page's decoder gives it (NaN codes as the
 * quiet NaN 0x7FC00000), optionally rounded to bf16 (nearest even).  Positions t >= seq_lens[b]
 * (clamped to capacity) are written as 0.
 *
 *   which   : 0 = K, 1 = V
 *   out     : device [B, KVH, out_len, D] of out_dtype
 * Errors: INVALID_ARG, OUT_OF_RANGE (out_len beyond capacity), HIP.
 */
kvq_status kvq_dequant(const kvq_cache* cache, int32_t which, const int32_t* seq_lens,
                       int32_t out_dtype, void* out, int32_t out_len, void* stream);

/*
 * Sliding-window attention (combs-models 0.2.2 src/kv.rs,
 * `KVCache::attention_opts` with `window`, and `attend`): a query at absolute
 * position p attends only to keys in (p - window, p]; older keys stay cached
 * but are masked out.  The window implies the causal bound.  window >= 1;
 * a window at least the sequence length gives the plain result.
 *
 * kvq_attention_decode_window / kvq_append_decode_window: as
 * kvq_attention_decode / kvq_append_decode, the query at position
 * seq_lens[b] - 1 seeing the last min(window, seq_lens[b]) tokens.
 * Workspace: kvq_workspace_size_window(cache, hint, 1, window).
 * kvq_attention_chunk_window: as kvq_attention_chunk with causal = 1, query i
 * at position ctx_lens[b] + i seeing keys in (ctx_lens[b] + i - window,
 * ctx_lens[b] + i].  Workspace: kvq_workspace_size_window(cache, hint + n, n,
 * window) (0 for the current kernel).
 * Errors: those of the plain entry points, plus INVALID_ARG for window < 1.
 * A sliding-window layer may keep only its window: give it a paged cache whose
 * block table maps each sequence's logical pages j onto P physical pages in
 * turn (j mod P), with 16 P >= window + n - 1 for appends of at most n rows.
 * Rows then overwrite rows that no later query sees; the loads of keys below
 * the window that the kernels still issue read finite, zero-weighted rows.
 */
kvq_status kvq_attention_decode_window(const kvq_cache* cache, const uint16_t* q, const int32_t* seq_lens,
                                       float attn_scale, int32_t window, uint16_t* out, void* workspace,
                                       size_t workspace_bytes, int32_t max_seq_len_hint, void* stream);
kvq_status kvq_append_decode_window(const kvq_cache* cache, const void* k_new, const void* v_new,
                                    int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens,
                                    float attn_scale, int32_t window, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, int32_t max_seq_len_hint, void* stream);
kvq_status kvq_attention_chunk_window(const kvq_cache* cache, const uint16_t* q, int32_t n,
                                      const int32_t* ctx_lens, float attn_scale, int32_t window, uint16_t* out,
                                      void* workspace, size_t workspace_bytes, int32_t max_ctx_len_hint,
                                      void* stream);
size_t kvq_workspace_size_window(const kvq_cache* cache, int32_t max_seq_len, int32_t n_query, int32_t window);

/*
 * Recent-window hybrid cache (abaddon 0.2.0-rc.1 src/kv_cache_quant_cuda.rs,
 * `OptimizedQuantizedKvCache` with `DynamicQuantConfig::unquantized_window`):
 * the last `window` positions of every sequence stay unquantized, as bf16,
 * in a ring beside the INT8 cache; older positions are INT8 in the cache
 * that the kvq_cache describes.  For a sequence of length L, position p is
 *   INT8, at its usual cache row,        if p <  L - window,
 *   bf16, in ring slot p % capacity,     if p >= L - window.
 * A row is quantized from its bf16 value: fp32 input rows are rounded to
 * bf16 (nearest even) when they enter, whichever call later moves them out
 * of the window.  capacity > window keeps the slot a fused step writes apart
 * from the slot it quantizes.
 */
typedef struct kvq_recent {
  int32_t window;    /* W >= 1 positions kept in bf16                         */
  int32_t capacity;  /* ring slots R per (sequence, KV head), R > W           */
  uint16_t* k;       /* device bf16 [batch, num_kv_heads, capacity, head_dim] */
  uint16_t* v;
} kvq_recent;

/*
 * kvq_append_recent — append n_new rows per sequence at the end of a hybrid
 * cache: start_pos[b] must be sequence b's current length (the caller's
 * contract).  With L' = start_pos[b] + n_new, the rows that leave the window
 * (old ring rows and new rows below L' - W) are quantized into the INT8
 * cache exactly as kvq_append would quantize their bf16 values, and the
 * rows at L' - W and above are stored, as bf16, in their ring slots
 * (`OptimizedQuantizedKvCache::append` steps).  Two launches: the rows
 * leaving the ring are quantized before any ring slot is overwritten.
 *
 *   k_new, v_new : device [B, KVH, n_new, D], fp32 or bf16 (in_dtype)
 * Errors: those of kvq_append, plus INVALID_ARG for a bad recent descriptor
 * (NULL, window < 1, capacity <= window, NULL ring pointers).
 */
kvq_status kvq_append_recent(const kvq_cache* cache, const kvq_recent* recent, const void* k_new,
                             const void* v_new, int32_t in_dtype, int32_t n_new,
                             const int32_t* start_pos, void* stream);

/*
 * kvq_attention_decode_recent — kvq_attention_decode over a hybrid cache:
 * each query attends to all seq_lens[b] tokens, the INT8 ones dequantized in
 * registers and the recent ones read as bf16 (the `get_kv` view: old rows
 * dequantized, then the recent rows).  The ring is one more split of the
 * split-K launch.  seq_lens[b] is clamped to [0, min(hint, capacity of the
 * INT8 cache)].  Workspace: kvq_workspace_size_recent(cache, recent, hint).
 * Head dims 64 and 128 run on the streaming kernel; the others on the
 * generic one, whose ring is a second loop after the INT8 rows.
 * Errors: those of kvq_attention_decode.
 */
kvq_status kvq_attention_decode_recent(const kvq_cache* cache, const kvq_recent* recent,
                                       const uint16_t* q, const int32_t* seq_lens, float attn_scale,
                                       uint16_t* out, void* workspace, size_t workspace_bytes,
                                       int32_t max_seq_len_hint, void* stream);

/*
 * kvq_append_decode_recent — one decode step on a hybrid cache in a single
 * launch: the new row of every sequence goes to position seq_lens[b] - 1
 * (its ring slot), the row leaving the window (position seq_lens[b] - 1 -
 * window, if any) is quantized into the INT8 cache, and the query attends
 * to all seq_lens[b] tokens: exactly kvq_append_recent (start_pos =
 * seq_lens - 1, n_new = 1) followed by kvq_attention_decode_recent.
 * Errors: those of both.
 */
kvq_status kvq_append_decode_recent(const kvq_cache* cache, const kvq_recent* recent,
                                    const void* k_new, const void* v_new, int32_t in_dtype,
                                    const uint16_t* q, const int32_t* seq_lens, float attn_scale,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    int32_t max_seq_len_hint, void* stream);

/*
 * kvq_dequant_recent — the `get_kv` view of one side of a hybrid cache:
 * out[b,h,t,:] is the dequantized INT8 row for t < L - W and the bf16 ring
 * row for L - W <= t < L (L = seq_lens[b] clamped to the INT8 capacity),
 * as fp32 or bf16; positions t >= L are 0.
 */
kvq_status kvq_dequant_recent(const kvq_cache* cache, const kvq_recent* recent, int32_t which,
                              const int32_t* seq_lens, int32_t out_dtype, void* out, int32_t out_len,
                              void* stream);

/*
 * kvq_attention_chunk_recent — chunked prefill over a hybrid cache: the n
 * chunk rows are already appended (kvq_append_recent), so the cache holds
 * L_b = ctx_lens[b] + n positions, INT8 below L_b - window and bf16 in the
 * ring from there.  Query i at position ctx_lens[b] + i sees keys
 * t <= ctx_lens[b] + i (bottom-right causal) of that `get_kv` view
 * (abaddon kv_cache_quant_cuda.rs `OptimizedQuantizedKvCache::get_kv`).
 * head_dim 64 and 128 (per-row scales, per-head block scales): one launch
 * of the MFMA chunk kernel, whose tiles hold both kinds of rows: INT8 rows
 * widened to exact f16 values as in kvq_attention_chunk, ring rows converted
 * to f16 with one power of two per row (exact for every element within
 * 2^28 of its row's largest), their own per-token factors beside them; no
 * workspace.  Other head dims and per-channel block scales: one decode per
 * (sequence, query) through the generic kernel, batch * n at most 65535.
 *   q, out, ctx_lens, max_ctx_len_hint: as kvq_attention_chunk; ctx_lens[b]
 *              must not exceed the hint (at head_dim 64 and 128 a larger
 *              length is taken as the hint)
 *   workspace: kvq_workspace_size_chunk_recent(cache, recent,
 *              max_ctx_len_hint + n, n) bytes (0 on the MFMA path)
 * Errors: those of kvq_attention_chunk, plus the recent descriptor's.
 */
kvq_status kvq_attention_chunk_recent(const kvq_cache* cache, const kvq_recent* recent, const uint16_t* q,
                                      int32_t n, const int32_t* ctx_lens, float attn_scale, uint16_t* out,
                                      void* workspace, size_t workspace_bytes, int32_t max_ctx_len_hint,
                                      void* stream);

/* Workspace bytes needed by kvq_attention_chunk_recent for n_query queries
 * per sequence and max_seq_len = hint + n (0 on an invalid descriptor or
 * argument). */
size_t kvq_workspace_size_chunk_recent(const kvq_cache* cache, const kvq_recent* recent, int32_t max_seq_len,
                                       int32_t n_query);

/* Workspace bytes needed by kvq_attention_decode_recent and
 * kvq_append_decode_recent for lengths up to max_seq_len (0 on an invalid
 * descriptor).  Like every sizing call it reads only the geometry: the
 * device pointers may still be NULL. */
size_t kvq_workspace_size_recent(const kvq_cache* cache, const kvq_recent* recent, int32_t max_seq_len);

/* Workspace bytes needed by kvq_attention_decode (n_query = 1) or
 * kvq_attention_chunk (n_query = chunk length) for lengths up to
 * max_seq_len.  0 on an invalid descriptor (see kvq_last_error).  Only the
 * geometry is read: the device pointers may still be NULL. */
size_t kvq_workspace_size(const kvq_cache* cache, int32_t max_seq_len, int32_t n_query);

/* Bytes of codes plus scales the descriptor addresses, K and V together
 * (realizar kv_cache_q8_init.rs `kv_cache_q8_memory_bytes`: 2 * (values +
 * 4 * scales) per layer; 2 bytes per scale in KVQ_SCALE_PER_TOKEN_BF16).
 * Contiguous: batch*KVH*max_len rows; paged: num_pages*KVH*16 rows.  0 on an
 * invalid descriptor.  Only the geometry is read, so a cache can be sized
 * before it is allocated (NULL pointers are accepted). */
uint64_t kvq_cache_bytes(const kvq_cache* cache);

/*
 * kvq_append_decode_noalloc — kvq_append_decode for callers that cannot
 * allocate or own device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same launch and kernels, with
 * the split counters and partials in a static device array of 8 MiB that
 * the library holds on each GPU it runs on until the process ends.  The
 * caller passes inputs and outputs only; no workspace argument, and the
 * call allocates nothing.  The array's address on a device is looked up at
 * the first call on that device, which also clears the array on `stream`
 * ahead of its own kernel; every completed call leaves it zero again.  All
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must not be made.
 *
 *   arguments : as kvq_append_decode, without workspace / workspace_bytes
 * Errors: those of kvq_append_decode; WORKSPACE when the call's counters
 * (4 * batch * head groups bytes) exceed the 64 KiB counter region or its
 * split partials (batch * num_heads * splits * (head_dim + 2) * 4 bytes)
 * exceed the rest of the array; HIP if the array's address cannot be
 * obtained.
 */
kvq_status kvq_append_decode_noalloc(const kvq_cache* cache, const void* k_new, const void* v_new,
                                     int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens,
                                     float attn_scale, uint16_t* out, int32_t max_seq_len_hint, void* stream);

/*
 * kvq_stream_read — measurement aid, not a step of the method: reads `bytes`
 * bytes of the device buffer `src` with 16-byte vector loads and does nothing
 * else with them (their xor is written to sink[0] only if it equals a fixed
 * constant, so the loads cannot be dropped).  Its rate is the read-bandwidth
 * ceiling that the attention kernels' achieved HBM bandwidth is compared
 * with.  `workgroups` workgroups of `waves_per_wg` (1..16) waves; each wave
 * keeps `depth` (1, 2, 4 or 8) to 2*depth 1-KB loads in flight.  interleave
 * is a set of flags: bit 0 set, the waves of a workgroup take turns over its
 * contiguous range, else each wave reads a contiguous range of its own; bit
 * 1 set, the loads are non-temporal (as the decode kernels' loads of K and V
 * codes); other bits set is INVALID_ARG.
 *   src  : device, 16-byte aligned, bytes a positive multiple of 16
 *   sink : device uint32 [1]
 * Errors: INVALID_ARG, HIP.
 */
kvq_status kvq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                           int32_t waves_per_wg, int32_t depth, int32_t interleave, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kvq_last_error(void);

/* Library version string. */
const char* kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
