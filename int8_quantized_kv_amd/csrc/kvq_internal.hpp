// Host-side declarations shared by the libkvq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_device.hpp"

namespace kvq {

// Records `msg` as this thread's last error and returns `st`.
kvq_status fail(kvq_status st, const char* fmt, ...);

inline CacheGeom geom_of(const kvq_cache& c) {
  CacheGeom g;
  g.kvh = c.num_kv_heads;
  g.max_len = c.max_len;
  g.paged = c.layout == KVQ_LAYOUT_PAGED ? 1 : 0;
  g.num_pages = c.num_pages;
  g.max_blocks = c.max_blocks_per_seq;
  g.block_table = c.block_table;
  return g;
}

inline bool is_fp8(const kvq_cache& c) {
  return c.scale_mode == KVQ_CODES_FP8_E4M3 || c.scale_mode == KVQ_CODES_FP8_E5M2;
}

// 0 for INT8 codes, 1 for FP8 E4M3, 2 for FP8 E5M2.
inline int fp8_kind(const kvq_cache& c) {
  return c.scale_mode == KVQ_CODES_FP8_E4M3 ? 1 : (c.scale_mode == KVQ_CODES_FP8_E5M2 ? 2 : 0);
}

// Block scales (per head or per channel over position-aligned blocks of
// kBlockRows rows of one sequence and KV head; hybrid caches only).
constexpr int kBlockRows = 16;
inline bool is_block_mode(const kvq_cache& c) {
  return c.scale_mode == KVQ_SCALE_BLOCK_HEAD || c.scale_mode == KVQ_SCALE_BLOCK_CHANNEL;
}

// The scale mode the attention and dequant kernels see: per-head block
// scales are stored once per row, so they read as per-token scales.
inline int kernel_scale_mode(const kvq_cache& c) {
  return c.scale_mode == KVQ_SCALE_BLOCK_HEAD ? KVQ_SCALE_PER_TOKEN : c.scale_mode;
}

// Scales per row: 1 per token (per-head blocks store theirs on every row),
// head_dim / 32 for group-32, none for FP8 codes; per-channel blocks hold
// head_dim scales per 16 rows, head_dim / 16 per row on average (their
// kernels index them per block, not through this count).
inline int scales_per_row(const kvq_cache& c) {
  if (c.scale_mode == KVQ_SCALE_BLOCK_CHANNEL) return c.head_dim / kBlockRows;
  return c.scale_mode == KVQ_SCALE_GROUP32 ? c.head_dim / 32 : (is_fp8(c) ? 0 : 1);
}

inline int scale_bytes(const kvq_cache& c) { return c.scale_mode == KVQ_SCALE_PER_TOKEN_BF16 ? 2 : 4; }

inline int capacity_of(const kvq_cache& c) {
  return c.layout == KVQ_LAYOUT_PAGED ? c.max_blocks_per_seq * kPageSize : c.max_len;
}

// Recent window of a hybrid cache (window 0: none).
struct RecentGeom {
  int32_t window = 0;
  int32_t cap = 0;       // ring slots per (sequence, KV head)
  uint16_t* k = nullptr; // bf16 [B, KVH, cap, D]
  uint16_t* v = nullptr;
};

inline RecentGeom recent_of(const kvq_recent* r) {
  RecentGeom g;
  if (r) {
    g.window = r->window;
    g.cap = r->capacity;
    g.k = r->k;
    g.v = r->v;
  }
  return g;
}

// ---- append / dequant -------------------------------------------------------
// pos_from_lens: start_pos holds seq_lens and the single new row goes to
// position seq_lens[b] - 1.  With a recent window the rows leaving it are
// quantized first (a launch of its own), then the new rows go to the INT8
// cache or the ring.
kvq_status launch_append(const kvq_cache& c, const void* k_new, const void* v_new, int in_dtype,
                         int n_new, const int32_t* start_pos, hipStream_t stream, bool pos_from_lens = false,
                         const RecentGeom& rc = RecentGeom());
kvq_status launch_dequant(const kvq_cache& c, int which, const int32_t* seq_lens, int out_dtype,
                          void* out, int out_len, hipStream_t stream, const RecentGeom& rc = RecentGeom());

// ---- decode -----------------------------------------------------------------
struct DecodePlan {
  int heads_per_wg;   // query heads sharing one K/V read (a divisor of H/KVH)
  int split_len;      // tokens per split (multiple of the kernel's pass size)
  int num_splits;     // splits per sequence for the hinted length
  bool longest_first; // workgroups take sequences in order of decreasing length
  size_t counter_bytes;  // leading bytes of the workspace holding split counters
  size_t workspace;   // bytes of counters + split partials
};
bool decode_supported(int head_dim);
// With a recent window the INT8 splits cover at most max_seq_len - window
// tokens; the last one's workgroup also attends to the ring.
// A sliding window (> 0) bounds each sequence's range to about the window.
// generic: plan for the generic kernel at any head size (chunk rows).
DecodePlan plan_decode(const kvq_cache& c, int max_seq_len, const RecentGeom& rc = RecentGeom(), int window = 0,
                       bool generic = false);
// new_k / new_v non-null: fused append of one row per sequence at position
// seq_lens[b] - 1 before the attention.
kvq_status launch_decode(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q,
                         const int32_t* seq_lens, float attn_scale, uint16_t* out, void* ws,
                         int max_seq_len, hipStream_t stream, const void* new_k = nullptr,
                         const void* new_v = nullptr, int new_dtype = KVQ_DT_BF16,
                         const RecentGeom& rc = RecentGeom(), int window = 0);

// ---- chunked prefill --------------------------------------------------------
bool chunk_supported(int head_dim);
size_t chunk_workspace(const kvq_cache& c, int max_total_len, int n);
// Head sizes the MFMA chunk kernel does not take (32, 96-224), per-channel
// block scales, and chunks over a recent-window cache at head sizes other
// than 64 and 128, go through the decode path's generic kernel, one grid row
// per (sequence, query), with split partials in the workspace.
bool chunk_generic_supported(int head_dim);
DecodePlan plan_chunk_generic(const kvq_cache& c, int max_total_len, int n, int window);
kvq_status launch_chunk_generic(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q, int n,
                                const int32_t* ctx_lens, int causal, float attn_scale, uint16_t* out, void* ws,
                                int max_total_len, hipStream_t stream, int window,
                                const RecentGeom& rc = RecentGeom());
// window > 0: sliding window (implies causal).  ring non-null: a hybrid
// cache (causal): keys below L - W are INT8 rows, the last W of each
// sequence's L0 + n rows are bf16 rows in their ring slots, and the kernel
// stages both kinds in its tiles (ctx_lens clamped to max_ctx_len).
kvq_status launch_chunk(const kvq_cache& c, const uint16_t* q, int n, const int32_t* ctx_lens,
                        int causal, float attn_scale, uint16_t* out, void* ws, int max_ctx_len,
                        hipStream_t stream, int window = 0, const RecentGeom* ring = nullptr);

}  // namespace kvq
