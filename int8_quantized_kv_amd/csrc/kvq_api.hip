// C ABI entry points of libkvq: argument validation, launch planning and the
// thread-local error message.  No allocation, no synchronisation, no device
// reads on the host (except in a KVQ_DEBUG build, below).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cmath>
#include <mutex>
#include <vector>

#include "kvq_internal.hpp"

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace kvq {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

namespace {

#ifdef KVQ_DEBUG
// Debug builds (-DKVQ_DEBUG) check the device-side values that the kernels
// take on trust and would otherwise clamp: every length within its bound
// and, in the paged layout, every page the call reads mapped to an arena
// page.  The check waits for the stream and copies the lengths and the block
// table to the host, so it is a testing aid, not for production.
//   lens  : device [batch]; total length of sequence b = lens[b] + add
//   bound : largest total length allowed (the hint, within the capacity)
//   rwin  : recent-window rows at the end of each sequence (not in pages)
//   first : tokens the earliest query sees before its own position under a
//           sliding window (window - 1), or -1 for every earlier token
kvq_status debug_check(const kvq_cache& c, const int32_t* lens, int32_t add, int64_t bound, int32_t rwin,
                       int32_t nq, int32_t first, hipStream_t stream, const char* who) {
  std::vector<int32_t> L(c.batch);
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(L.data(), lens, sizeof(int32_t) * c.batch, hipMemcpyDeviceToHost);
  std::vector<int32_t> bt;
  const bool paged = c.layout == KVQ_LAYOUT_PAGED;
  if (e == hipSuccess && paged) {
    bt.resize(static_cast<size_t>(c.batch) * c.max_blocks_per_seq);
    e = hipMemcpy(bt.data(), c.block_table, sizeof(int32_t) * bt.size(), hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: debug check: copy failed: %s", who, hipGetErrorString(e));
  for (int b = 0; b < c.batch; ++b) {
    const int64_t total = static_cast<int64_t>(L[b]) + add;
    if (L[b] < 0 || total > bound)
      return fail(KVQ_ERR_OUT_OF_RANGE, "%s: debug check: sequence %d has length %lld, outside [0, %lld]", who, b,
                  static_cast<long long>(total), static_cast<long long>(bound));
    if (!paged) continue;
    const int64_t hi = total - rwin > 0 ? total - rwin : 0;  // INT8 positions [lo, hi) are read
    int64_t lo = first >= 0 ? total - nq - first : 0;
    if (lo < 0) lo = 0;
    for (int64_t pos = lo & ~static_cast<int64_t>(kPageSize - 1); pos < hi; pos += kPageSize) {
      const int64_t blk = pos / kPageSize;
      const int32_t id = blk < c.max_blocks_per_seq ? bt[static_cast<size_t>(b) * c.max_blocks_per_seq + blk] : -1;
      if (id < 0 || id >= c.num_pages)
        return fail(KVQ_ERR_OUT_OF_RANGE, "%s: debug check: sequence %d position %lld is in page %d, outside [0, %d)",
                    who, b, static_cast<long long>(pos), id, c.num_pages);
    }
  }
  return KVQ_OK;
}
#endif

// Descriptor checks common to every entry point.
// The descriptor's geometry, and with need_pointers its device pointers (the
// sizing calls take descriptors of caches not allocated yet).
kvq_status check_cache(const kvq_cache* c, const char* who, bool need_pointers = true) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "%s: cache descriptor is NULL", who);
  if (c->batch <= 0 || c->num_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "%s: batch, num_heads, num_kv_heads and head_dim must be positive", who);
  if (c->num_heads % c->num_kv_heads != 0)
    return fail(KVQ_ERR_INVALID_ARG, "%s: num_heads (%d) must be a multiple of num_kv_heads (%d)", who,
                c->num_heads, c->num_kv_heads);
  if (c->head_dim % 32 != 0)
    return fail(KVQ_ERR_INVALID_ARG, "%s: head_dim (%d) must be a multiple of 32", who, c->head_dim);
  if (c->head_dim > 256)
    return fail(KVQ_ERR_INVALID_ARG, "%s: head_dim (%d) must be at most 256", who, c->head_dim);
  if (c->scale_mode < KVQ_SCALE_PER_TOKEN || c->scale_mode > KVQ_SCALE_BLOCK_CHANNEL)
    return fail(KVQ_ERR_INVALID_ARG, "%s: unknown scale_mode %d", who, c->scale_mode);
  if (c->layout == KVQ_LAYOUT_CONTIGUOUS) {
    if (c->max_len <= 0) return fail(KVQ_ERR_INVALID_ARG, "%s: contiguous cache needs max_len > 0", who);
    if (is_block_mode(*c) && c->max_len % kBlockRows != 0)
      return fail(KVQ_ERR_INVALID_ARG, "%s: block scales need max_len %% %d == 0 (got %d)", who, kBlockRows,
                  c->max_len);
  } else if (c->layout == KVQ_LAYOUT_PAGED) {
    if (c->page_size != kPageSize)
      return fail(KVQ_ERR_INVALID_ARG, "%s: page_size must be %d (got %d)", who, kPageSize, c->page_size);
    if (c->num_pages <= 0 || c->max_blocks_per_seq <= 0)
      return fail(KVQ_ERR_INVALID_ARG, "%s: paged cache needs num_pages > 0 and max_blocks_per_seq > 0", who);
    if (need_pointers && !c->block_table) return fail(KVQ_ERR_INVALID_ARG, "%s: paged cache needs a block_table", who);
    if (static_cast<int64_t>(c->max_blocks_per_seq) * kPageSize > 0x7fffffffLL)
      return fail(KVQ_ERR_INVALID_ARG, "%s: max_blocks_per_seq too large", who);
  } else {
    return fail(KVQ_ERR_INVALID_ARG, "%s: unknown layout %d", who, c->layout);
  }
  if (!need_pointers) return KVQ_OK;
  if (!c->k_codes || !c->v_codes) return fail(KVQ_ERR_INVALID_ARG, "%s: cache code pointers must be non-NULL", who);
  if (!is_fp8(*c)) {  // FP8 codes carry no scales
    if (!c->k_scales || !c->v_scales)
      return fail(KVQ_ERR_INVALID_ARG, "%s: cache scale pointers must be non-NULL", who);
    if (((reinterpret_cast<uintptr_t>(c->k_scales) | reinterpret_cast<uintptr_t>(c->v_scales)) & 3) != 0)
      return fail(KVQ_ERR_INVALID_ARG, "%s: scale arrays must be 4-byte aligned", who);
  }
  return KVQ_OK;
}

kvq_status check_split_workspace(size_t need, void* ws, size_t ws_bytes, const char* who) {
  if (need == 0) return KVQ_OK;
  if (!ws) return fail(KVQ_ERR_WORKSPACE, "%s: workspace is NULL but %zu bytes are needed", who, need);
  if (ws_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu bytes needed", who,
                ws_bytes, need);
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

KVQ_API const char* kvq_last_error(void) { return g_err; }

KVQ_API const char* kvq_version(void) { return "kvq 0.1.0 (gfx950)"; }

KVQ_API uint64_t kvq_cache_bytes(const kvq_cache* c) {
  g_err[0] = '\0';
  if (check_cache(c, "kvq_cache_bytes", false) != KVQ_OK) return 0;
  const uint64_t rows = c->layout == KVQ_LAYOUT_PAGED
                            ? static_cast<uint64_t>(c->num_pages) * c->num_kv_heads * kPageSize
                            : static_cast<uint64_t>(c->batch) * c->num_kv_heads * c->max_len;
  const uint64_t per_row = static_cast<uint64_t>(c->head_dim) + static_cast<uint64_t>(scale_bytes(*c)) * scales_per_row(*c);
  return 2ull * rows * per_row;
}

namespace kvq {
namespace {

kvq_status check_recent(const kvq_recent* r, const kvq_cache& c, const char* who, bool need_pointers = true) {
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  if (r->window < 1) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, r->window);
  if (r->capacity <= r->window)
    return fail(KVQ_ERR_INVALID_ARG, "%s: ring capacity (%d) must exceed the window (%d)", who, r->capacity,
                r->window);
  if (static_cast<int64_t>(r->capacity) * c.head_dim > 0x7fffffffLL)
    return fail(KVQ_ERR_INVALID_ARG, "%s: ring capacity too large", who);
  if (need_pointers && (!r->k || !r->v)) return fail(KVQ_ERR_INVALID_ARG, "%s: ring pointers must be non-NULL", who);
  if (is_fp8(c)) return fail(KVQ_ERR_UNSUPPORTED, "%s: a recent window over FP8 codes is not supported", who);
  if (is_block_mode(c) && r->window < kBlockRows - 1)
    return fail(KVQ_ERR_INVALID_ARG, "%s: block scales need a window of at least %d (got %d)", who, kBlockRows - 1,
                r->window);
  return KVQ_OK;
}

// Block scales exist only on hybrid caches (a block is quantized when its
// first row leaves the recent window).
kvq_status check_block_needs_recent(const kvq_cache& c, const kvq_recent* r, const char* who) {
  if (is_block_mode(c) && !r)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: block scale modes need a recent-window cache (the kvq_*_recent calls)",
                who);
  return KVQ_OK;
}

bool finite(float x) { return x == x && x != INFINITY && x != -INFINITY; }

// On a hybrid cache the MFMA chunk kernel (with the ring kernel) takes head
// dims 64 and 128 in every per-row scale mode; other head dims and
// per-channel block scales go through the generic kernel.
bool mfma_hybrid_ok(const kvq_cache& c) {
  return (c.head_dim == 64 || c.head_dim == 128) && c.scale_mode != KVQ_SCALE_BLOCK_CHANNEL;
}

size_t workspace_impl(const kvq_cache* c, const kvq_recent* r, int32_t max_seq_len, int32_t n_query,
                      const char* who, int32_t window = 0) {
  g_err[0] = '\0';
  if (check_cache(c, who, false) != KVQ_OK) return 0;
  if (r && check_recent(r, *c, who, false) != KVQ_OK) return 0;
  if (check_block_needs_recent(*c, r, who) != KVQ_OK) return 0;
  if (max_seq_len <= 0 || n_query <= 0) {
    fail(KVQ_ERR_INVALID_ARG, "%s: max_seq_len and n_query must be positive", who);
    return 0;
  }
  if (n_query == 1) {
    // one query: a decode, or a one-row chunk, which at head dims without an
    // MFMA chunk kernel runs on the generic kernel's (shorter) splits
    size_t w = plan_decode(*c, max_seq_len, recent_of(r), window).workspace;
    if (!r && !chunk_supported(c->head_dim) && chunk_generic_supported(c->head_dim)) {
      const size_t wc = plan_chunk_generic(*c, max_seq_len, 1, window).workspace;
      w = wc > w ? wc : w;
    }
    return w;
  }
  if (!chunk_supported(c->head_dim) && chunk_generic_supported(c->head_dim))
    return plan_chunk_generic(*c, max_seq_len, n_query, window).workspace;
  return chunk_workspace(*c, max_seq_len, n_query);
}

kvq_status append_impl(const kvq_cache* c, const kvq_recent* r, const void* k_new, const void* v_new,
                       int32_t in_dtype, int32_t n_new, const int32_t* start_pos, void* stream, const char* who) {
  kvq_status st = check_cache(c, who);
  if (st != KVQ_OK) return st;
  if (r && (st = check_recent(r, *c, who)) != KVQ_OK) return st;
  if ((st = check_block_needs_recent(*c, r, who)) != KVQ_OK) return st;
  if (!k_new || !v_new || !start_pos) return fail(KVQ_ERR_INVALID_ARG, "%s: k_new, v_new and start_pos must be non-NULL", who);
  if (in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16)
    return fail(KVQ_ERR_INVALID_ARG, "%s: in_dtype must be KVQ_DT_F32 or KVQ_DT_BF16", who);
  if (n_new <= 0) return fail(KVQ_ERR_INVALID_ARG, "%s: n_new must be positive (got %d)", who, n_new);
  if (n_new > capacity_of(*c))
    return fail(KVQ_ERR_OUT_OF_RANGE, "%s: n_new (%d) exceeds the per-sequence capacity (%d)", who, n_new,
                capacity_of(*c));
  return launch_append(*c, k_new, v_new, in_dtype, n_new, start_pos, static_cast<hipStream_t>(stream), false,
                       recent_of(r));
}

// Decode, plain or fused (k_new non-NULL), with or without a recent window.
kvq_status decode_impl(const kvq_cache* c, const kvq_recent* r, bool fused, const void* k_new, const void* v_new,
                       int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens, float attn_scale,
                       uint16_t* out, void* workspace, size_t workspace_bytes, int32_t max_seq_len_hint,
                       void* stream, const char* who, int32_t window = 0) {
  kvq_status st = check_cache(c, who);
  if (st != KVQ_OK) return st;
  if (r && (st = check_recent(r, *c, who)) != KVQ_OK) return st;
  if ((st = check_block_needs_recent(*c, r, who)) != KVQ_OK) return st;
  if (window < 0) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, window);
  if (fused) {
    if (!k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "%s: k_new and v_new must be non-NULL", who);
    if (in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16)
      return fail(KVQ_ERR_INVALID_ARG, "%s: in_dtype must be KVQ_DT_F32 or KVQ_DT_BF16", who);
  }
  if (!q || !seq_lens || !out) return fail(KVQ_ERR_INVALID_ARG, "%s: q, seq_lens and out must be non-NULL", who);
  if (!finite(attn_scale)) return fail(KVQ_ERR_INVALID_ARG, "%s: attn_scale must be finite", who);
  if (max_seq_len_hint < 1 || max_seq_len_hint > capacity_of(*c))
    return fail(KVQ_ERR_OUT_OF_RANGE, "%s: max_seq_len_hint (%d) must be in [1, %d]", who, max_seq_len_hint,
                capacity_of(*c));
  if (!decode_supported(c->head_dim))
    return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d not supported (multiples of 32 up to 256)", who, c->head_dim);
  const RecentGeom rc = recent_of(r);
  const DecodePlan plan = plan_decode(*c, max_seq_len_hint, rc, window);
  st = check_split_workspace(plan.workspace, workspace, workspace_bytes, who);
  if (st != KVQ_OK) return st;
#ifdef KVQ_DEBUG
  st = debug_check(*c, seq_lens, 0, max_seq_len_hint, rc.window, 1, window > 0 ? window - 1 : -1,
                   static_cast<hipStream_t>(stream), who);
  if (st != KVQ_OK) return st;
#endif
  return launch_decode(*c, plan, q, seq_lens, attn_scale, out, workspace, max_seq_len_hint,
                       static_cast<hipStream_t>(stream), fused ? k_new : nullptr, fused ? v_new : nullptr,
                       in_dtype, rc, window);
}

kvq_status dequant_impl(const kvq_cache* c, const kvq_recent* r, int32_t which, const int32_t* seq_lens,
                        int32_t out_dtype, void* out, int32_t out_len, void* stream, const char* who) {
  kvq_status st = check_cache(c, who);
  if (st != KVQ_OK) return st;
  if (r && (st = check_recent(r, *c, who)) != KVQ_OK) return st;
  if ((st = check_block_needs_recent(*c, r, who)) != KVQ_OK) return st;
  if (which != 0 && which != 1) return fail(KVQ_ERR_INVALID_ARG, "%s: which must be 0 (K) or 1 (V)", who);
  if (!seq_lens || !out) return fail(KVQ_ERR_INVALID_ARG, "%s: seq_lens and out must be non-NULL", who);
  if (out_dtype != KVQ_DT_F32 && out_dtype != KVQ_DT_BF16)
    return fail(KVQ_ERR_INVALID_ARG, "%s: out_dtype must be KVQ_DT_F32 or KVQ_DT_BF16", who);
  if (out_len <= 0 || out_len > capacity_of(*c))
    return fail(KVQ_ERR_OUT_OF_RANGE, "%s: out_len (%d) must be in [1, %d]", who, out_len, capacity_of(*c));
  return launch_dequant(*c, which, seq_lens, out_dtype, out, out_len, static_cast<hipStream_t>(stream),
                        recent_of(r));
}

}  // namespace
}  // namespace kvq

KVQ_API size_t kvq_workspace_size(const kvq_cache* c, int32_t max_seq_len, int32_t n_query) {
  return workspace_impl(c, nullptr, max_seq_len, n_query, "kvq_workspace_size");
}

KVQ_API size_t kvq_workspace_size_recent(const kvq_cache* c, const kvq_recent* r, int32_t max_seq_len) {
  if (!r) {
    fail(KVQ_ERR_INVALID_ARG, "kvq_workspace_size_recent: recent-window descriptor is NULL");
    return 0;
  }
  return workspace_impl(c, r, max_seq_len, 1, "kvq_workspace_size_recent");
}

KVQ_API kvq_status kvq_append(const kvq_cache* c, const void* k_new, const void* v_new, int32_t in_dtype,
                              int32_t n_new, const int32_t* start_pos, void* stream) {
  return append_impl(c, nullptr, k_new, v_new, in_dtype, n_new, start_pos, stream, "kvq_append");
}

KVQ_API kvq_status kvq_append_recent(const kvq_cache* c, const kvq_recent* r, const void* k_new, const void* v_new,
                                     int32_t in_dtype, int32_t n_new, const int32_t* start_pos, void* stream) {
  const char* who = "kvq_append_recent";
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  return append_impl(c, r, k_new, v_new, in_dtype, n_new, start_pos, stream, who);
}

KVQ_API kvq_status kvq_attention_decode(const kvq_cache* c, const uint16_t* q, const int32_t* seq_lens,
                                        float attn_scale, uint16_t* out, void* workspace,
                                        size_t workspace_bytes, int32_t max_seq_len_hint, void* stream) {
  return decode_impl(c, nullptr, false, nullptr, nullptr, KVQ_DT_BF16, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, "kvq_attention_decode");
}

KVQ_API kvq_status kvq_attention_decode_recent(const kvq_cache* c, const kvq_recent* r, const uint16_t* q,
                                               const int32_t* seq_lens, float attn_scale, uint16_t* out,
                                               void* workspace, size_t workspace_bytes, int32_t max_seq_len_hint,
                                               void* stream) {
  const char* who = "kvq_attention_decode_recent";
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  return decode_impl(c, r, false, nullptr, nullptr, KVQ_DT_BF16, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, who);
}

KVQ_API kvq_status kvq_append_decode(const kvq_cache* c, const void* k_new, const void* v_new, int32_t in_dtype,
                                     const uint16_t* q, const int32_t* seq_lens, float attn_scale, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, int32_t max_seq_len_hint,
                                     void* stream) {
  return decode_impl(c, nullptr, true, k_new, v_new, in_dtype, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, "kvq_append_decode");
}

KVQ_API kvq_status kvq_append_decode_recent(const kvq_cache* c, const kvq_recent* r, const void* k_new,
                                            const void* v_new, int32_t in_dtype, const uint16_t* q,
                                            const int32_t* seq_lens, float attn_scale, uint16_t* out,
                                            void* workspace, size_t workspace_bytes, int32_t max_seq_len_hint,
                                            void* stream) {
  const char* who = "kvq_append_decode_recent";
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  return decode_impl(c, r, true, k_new, v_new, in_dtype, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, who);
}

// ---------------------------------------------------------------------------
// The fused decode step without a caller workspace: split counters and
// partials live in a static device array of kScratchBytes, one per GPU, held
// until the process ends.  Its address on each device comes from
// hipGetSymbolAddress at the first call on that device; host code never
// passes the array's own name to a kernel or a copy (on the host that name is
// a stand-in, not a device address).
// ---------------------------------------------------------------------------
namespace kvq {
namespace {

constexpr size_t kScratchBytes = 8u << 20;      // 8 MiB per GPU
constexpr size_t kScratchCounters = 64u << 10;  // fixed counter region at the front
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of this device's scratch array, looked up once per
// device (with that device current); the whole array is cleared on `stream`
// at that first call, ahead of the call's own kernel (every call leaves the
// counters and the partial words it used zero again).
kvq_status scratch_of(int dev, hipStream_t stream, void** out, const char* who) {
  ScratchSlot& s = g_scratch[dev];
  bool first = false;
  std::call_once(s.once, [&] {
    first = true;
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
  });
  if (s.err != hipSuccess || !s.ptr)
    return fail(KVQ_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", who, dev,
                hipGetErrorString(s.err));
  if (first) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(s.ptr),
                       static_cast<int>(kScratchBytes / 4));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: scratch clear failed: %s", who, hipGetErrorString(e));
  }
  *out = s.ptr;
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

KVQ_API kvq_status kvq_append_decode_noalloc(const kvq_cache* c, const void* k_new, const void* v_new,
                                             int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens,
                                             float attn_scale, uint16_t* out, int32_t max_seq_len_hint,
                                             void* stream) {
  const char* who = "kvq_append_decode_noalloc";
  kvq_status st = check_cache(c, who);
  if (st != KVQ_OK) return st;
  if ((st = check_block_needs_recent(*c, nullptr, who)) != KVQ_OK) return st;
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "%s: k_new and v_new must be non-NULL", who);
  if (in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16)
    return fail(KVQ_ERR_INVALID_ARG, "%s: in_dtype must be KVQ_DT_F32 or KVQ_DT_BF16", who);
  if (!q || !seq_lens || !out) return fail(KVQ_ERR_INVALID_ARG, "%s: q, seq_lens and out must be non-NULL", who);
  if (!finite(attn_scale)) return fail(KVQ_ERR_INVALID_ARG, "%s: attn_scale must be finite", who);
  if (max_seq_len_hint < 1 || max_seq_len_hint > capacity_of(*c))
    return fail(KVQ_ERR_OUT_OF_RANGE, "%s: max_seq_len_hint (%d) must be in [1, %d]", who, max_seq_len_hint,
                capacity_of(*c));
  if (!decode_supported(c->head_dim))
    return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d not supported (multiples of 32 up to 256)", who, c->head_dim);
  // the caller's plan, with the split counters moved to the fixed region at
  // the front of the array and the partials after it
  DecodePlan plan = plan_decode(*c, max_seq_len_hint);
  if (plan.counter_bytes > kScratchCounters)
    return fail(KVQ_ERR_WORKSPACE, "%s: %zu bytes of split counters exceed the %zu-byte counter region", who,
                plan.counter_bytes, kScratchCounters);
  const size_t need = plan.workspace - plan.counter_bytes + kScratchCounters;
  if (need > kScratchBytes)
    return fail(KVQ_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch, above the %zu-byte maximum "
                "(use kvq_append_decode with a workspace)", who, need, kScratchBytes);
  plan.counter_bytes = kScratchCounters;
  plan.workspace = need;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "%s: device %d beyond %d", who, dev, kMaxDevices);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_of(dev, hs, &ws, who);
  if (st != KVQ_OK) return st;
#ifdef KVQ_DEBUG
  st = debug_check(*c, seq_lens, 0, max_seq_len_hint, 0, 1, -1, hs, who);
  if (st != KVQ_OK) return st;
#endif
  return launch_decode(*c, plan, q, seq_lens, attn_scale, out, ws, max_seq_len_hint, hs, k_new, v_new, in_dtype);
}

namespace kvq {
namespace {

kvq_status chunk_impl(const kvq_cache* c, const uint16_t* q, int32_t n, const int32_t* ctx_lens, int32_t causal,
                      float attn_scale, int32_t window, uint16_t* out, void* workspace, size_t workspace_bytes,
                      int32_t max_ctx_len_hint, void* stream, const char* who, const kvq_recent* r = nullptr) {
  kvq_status st = check_cache(c, who);
  if (st != KVQ_OK) return st;
  if (r && (st = check_recent(r, *c, who)) != KVQ_OK) return st;
  if ((st = check_block_needs_recent(*c, r, who)) != KVQ_OK) return st;
  if (!q || !ctx_lens || !out) return fail(KVQ_ERR_INVALID_ARG, "%s: q, ctx_lens and out must be non-NULL", who);
  if (n <= 0) return fail(KVQ_ERR_INVALID_ARG, "%s: n must be positive (got %d)", who, n);
  if (window < 0) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, window);
  if (!finite(attn_scale)) return fail(KVQ_ERR_INVALID_ARG, "%s: attn_scale must be finite", who);
  if (max_ctx_len_hint < 0 || static_cast<int64_t>(max_ctx_len_hint) + n > capacity_of(*c))
    return fail(KVQ_ERR_OUT_OF_RANGE, "%s: max_ctx_len_hint + n (%lld) exceeds the capacity (%d)", who,
                static_cast<long long>(max_ctx_len_hint) + n, capacity_of(*c));
#ifdef KVQ_DEBUG
  st = debug_check(*c, ctx_lens, n, static_cast<int64_t>(max_ctx_len_hint) + n, r ? recent_of(r).window : 0, n,
                   window > 0 ? window - 1 : -1, static_cast<hipStream_t>(stream), who);
  if (st != KVQ_OK) return st;
#endif
  // a hybrid cache at an MFMA head size: the MFMA kernel stages INT8 rows and
  // bf16 ring rows in the same tiles (no workspace)
  if (r && mfma_hybrid_ok(*c)) {
    const RecentGeom rc = recent_of(r);
    return launch_chunk(*c, q, n, ctx_lens, 1, attn_scale, out, workspace, max_ctx_len_hint,
                        static_cast<hipStream_t>(stream), 0, &rc);
  }
  // head dims without an MFMA chunk kernel go through the generic kernel
  if (r || !chunk_supported(c->head_dim)) {
    if (!chunk_supported(c->head_dim) && !chunk_generic_supported(c->head_dim))
      return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d not supported", who, c->head_dim);
    const DecodePlan plan = plan_chunk_generic(*c, max_ctx_len_hint + n, n, window);
    st = check_split_workspace(plan.workspace, workspace, workspace_bytes, who);
    if (st != KVQ_OK) return st;
    return launch_chunk_generic(*c, plan, q, n, ctx_lens, causal, attn_scale, out, workspace, max_ctx_len_hint + n,
                                static_cast<hipStream_t>(stream), window, recent_of(r));
  }
  st = check_split_workspace(chunk_workspace(*c, max_ctx_len_hint + n, n), workspace, workspace_bytes, who);
  if (st != KVQ_OK) return st;
  return launch_chunk(*c, q, n, ctx_lens, causal, attn_scale, out, workspace, max_ctx_len_hint,
                      static_cast<hipStream_t>(stream), window);
}

}  // namespace
}  // namespace kvq

KVQ_API kvq_status kvq_attention_chunk(const kvq_cache* c, const uint16_t* q, int32_t n, const int32_t* ctx_lens,
                                       int32_t causal, float attn_scale, uint16_t* out, void* workspace,
                                       size_t workspace_bytes, int32_t max_ctx_len_hint, void* stream) {
  return chunk_impl(c, q, n, ctx_lens, causal, attn_scale, 0, out, workspace, workspace_bytes, max_ctx_len_hint,
                    stream, "kvq_attention_chunk");
}

KVQ_API kvq_status kvq_attention_chunk_recent(const kvq_cache* c, const kvq_recent* r, const uint16_t* q, int32_t n,
                                              const int32_t* ctx_lens, float attn_scale, uint16_t* out,
                                              void* workspace, size_t workspace_bytes, int32_t max_ctx_len_hint,
                                              void* stream) {
  const char* who = "kvq_attention_chunk_recent";
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  return chunk_impl(c, q, n, ctx_lens, 1, attn_scale, 0, out, workspace, workspace_bytes, max_ctx_len_hint, stream,
                    who, r);
}

KVQ_API size_t kvq_workspace_size_chunk_recent(const kvq_cache* c, const kvq_recent* r, int32_t max_seq_len,
                                               int32_t n_query) {
  const char* who = "kvq_workspace_size_chunk_recent";
  g_err[0] = '\0';
  if (!r) {
    fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
    return 0;
  }
  if (check_cache(c, who, false) != KVQ_OK || check_recent(r, *c, who, false) != KVQ_OK) return 0;
  if (max_seq_len <= 0 || n_query <= 0) {
    fail(KVQ_ERR_INVALID_ARG, "%s: max_seq_len and n_query must be positive", who);
    return 0;
  }
  if (mfma_hybrid_ok(*c)) return 0;  // the MFMA kernel needs none
  return plan_chunk_generic(*c, max_seq_len, n_query, 0).workspace;
}

KVQ_API kvq_status kvq_attention_chunk_window(const kvq_cache* c, const uint16_t* q, int32_t n,
                                              const int32_t* ctx_lens, float attn_scale, int32_t window,
                                              uint16_t* out, void* workspace, size_t workspace_bytes,
                                              int32_t max_ctx_len_hint, void* stream) {
  const char* who = "kvq_attention_chunk_window";
  if (window < 1) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, window);
  return chunk_impl(c, q, n, ctx_lens, 1, attn_scale, window, out, workspace, workspace_bytes, max_ctx_len_hint,
                    stream, who);
}

KVQ_API kvq_status kvq_attention_decode_window(const kvq_cache* c, const uint16_t* q, const int32_t* seq_lens,
                                               float attn_scale, int32_t window, uint16_t* out, void* workspace,
                                               size_t workspace_bytes, int32_t max_seq_len_hint, void* stream) {
  const char* who = "kvq_attention_decode_window";
  if (window < 1) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, window);
  return decode_impl(c, nullptr, false, nullptr, nullptr, KVQ_DT_BF16, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, who, window);
}

KVQ_API kvq_status kvq_append_decode_window(const kvq_cache* c, const void* k_new, const void* v_new,
                                            int32_t in_dtype, const uint16_t* q, const int32_t* seq_lens,
                                            float attn_scale, int32_t window, uint16_t* out, void* workspace,
                                            size_t workspace_bytes, int32_t max_seq_len_hint, void* stream) {
  const char* who = "kvq_append_decode_window";
  if (window < 1) return fail(KVQ_ERR_INVALID_ARG, "%s: window must be at least 1 (got %d)", who, window);
  return decode_impl(c, nullptr, true, k_new, v_new, in_dtype, q, seq_lens, attn_scale, out, workspace,
                     workspace_bytes, max_seq_len_hint, stream, who, window);
}

KVQ_API size_t kvq_workspace_size_window(const kvq_cache* c, int32_t max_seq_len, int32_t n_query, int32_t window) {
  if (window < 1) {
    fail(KVQ_ERR_INVALID_ARG, "kvq_workspace_size_window: window must be at least 1 (got %d)", window);
    return 0;
  }
  return workspace_impl(c, nullptr, max_seq_len, n_query, "kvq_workspace_size_window", window);
}

KVQ_API kvq_status kvq_dequant(const kvq_cache* c, int32_t which, const int32_t* seq_lens, int32_t out_dtype,
                               void* out, int32_t out_len, void* stream) {
  return dequant_impl(c, nullptr, which, seq_lens, out_dtype, out, out_len, stream, "kvq_dequant");
}

KVQ_API kvq_status kvq_dequant_recent(const kvq_cache* c, const kvq_recent* r, int32_t which,
                                      const int32_t* seq_lens, int32_t out_dtype, void* out, int32_t out_len,
                                      void* stream) {
  const char* who = "kvq_dequant_recent";
  if (!r) return fail(KVQ_ERR_INVALID_ARG, "%s: recent-window descriptor is NULL", who);
  return dequant_impl(c, r, which, seq_lens, out_dtype, out, out_len, stream, who);
}
