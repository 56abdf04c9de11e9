// Decode attention: the generic kernel (decode at head_dim 256, chunk rows
// the MFMA chunk kernel does not take) and its merge, the split planner, and
// the launch of both kernels.  The streaming kernel lives in
// kvq_decode_stream.hpp.
#include "kvq_decode_generic.hpp"

namespace kvq {
namespace {

// Log-sum-exp merge of the split partials of one (sequence, head); bf16 out.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int D) {
  const int h = blockIdx.x;
  const int v = blockIdx.y;
  int b, qi;
  const int L = row_len(p, v, b, qi);
  const int nq = p.chunk_n > 0 ? p.chunk_n : 1;
  const int H = p.num_heads;
  const int t_lo = p.window > 0 ? max(L - p.window, 0) : 0;  // the splits start at the window
  const int ns = split_count(L - t_lo, p.split_len);
  const int64_t base = (static_cast<int64_t>(v) * H + h) * p.num_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_ml[(base + s) * 2]);
  float den = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float ms = p.part_ml[(base + s) * 2];
    if (ms != -INFINITY) den = fmaf(p.part_ml[(base + s) * 2 + 1], exp2f(ms - M), den);
  }
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float num = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float ms = p.part_ml[(base + s) * 2];
      if (ms != -INFINITY) num = fmaf(p.part_o[(base + s) * D + d], exp2f(ms - M), num);
      p.part_o[(base + s) * D + d] = 0.0f;  // the workspace goes back to zero
    }
    const float val = den > 0.0f ? num / den : 0.0f;
    p.out[((static_cast<int64_t>(b) * H + h) * nq + qi) * D + d] = f32_to_bf16_rne(val);
  }
  __syncthreads();  // every thread has read the (m, l) pairs
  for (int s = threadIdx.x; s < ns; s += blockDim.x) {
    p.part_ml[(base + s) * 2] = 0.0f;
    p.part_ml[(base + s) * 2 + 1] = 0.0f;
  }
}

int heads_per_wg(int gqa) {
  if (gqa % 4 == 0) return 4;
  if (gqa % 2 == 0) return 2;
  return 1;
}

bool use_stream(int head_dim) { return head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256; }

// The streaming kernel takes head dims 32, 64, 128 and 256 in every per-row
// scale mode; per-channel block scales, and head dim 256 with a recent window
// (whose ring pass holds two dims per lane), run on the generic kernel.
bool stream_ok(const kvq_cache& c, const RecentGeom& rc) {
  return use_stream(c.head_dim) && c.scale_mode != KVQ_SCALE_BLOCK_CHANNEL && !(c.head_dim == 256 && rc.window > 0);
}

int pass_tokens(int head_dim, bool stream_kernel) {
  // tokens a workgroup consumes per step: one 64-token block per wave for
  // the streaming kernel (two 32-token ones at head dims 128 and 256), one
  // pass of all waves for the generic kernel
  return stream_kernel ? kBlock * kStreamWaves : (kWave / (head_dim / 16)) * kWaves;
}

// The generic kernel at any supported head dim.
void launch_generic_any(int head_dim, int hpw, int sm, bool paged, const DecodeParams& p, dim3 grid,
                        hipStream_t st) {
  switch (head_dim) {
    case 32: launch_generic_all<32>(hpw, sm, paged, p, grid, st); break;
    case 64: launch_generic_all<64>(hpw, sm, paged, p, grid, st); break;
    case 128: launch_generic_all<128>(hpw, sm, paged, p, grid, st); break;
    case 256: launch_generic_all<256>(hpw, sm, paged, p, grid, st); break;
    default: launch_generic_wide(head_dim, hpw, sm, paged, p, grid, st); break;
  }
}

void launch_decode_kernel(int head_dim, bool stream_kernel, bool append, int hpw, int sm, bool paged,
                          const DecodeParams& p, dim3 grid, hipStream_t st) {
  if (stream_kernel) {
    if (sm == kSmGroup32) launch_stream_group32(head_dim, hpw, paged, append, p, grid, st);
    else if (sm == kSmTokenBf16) launch_stream_bf16(head_dim, hpw, paged, append, p, grid, st);
    else if (sm == kSmFp8E4M3 || sm == kSmFp8E5M2) launch_stream_fp8(head_dim, hpw, sm, paged, append, p, grid, st);
    else launch_stream_token(head_dim, hpw, paged, append, p, grid, st);
    return;
  }
  launch_generic_any(head_dim, hpw, sm, paged, p, grid, st);
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool decode_supported(int head_dim) { return head_dim % 32 == 0 && head_dim >= 32 && head_dim <= 256; }

DecodePlan plan_decode(const kvq_cache& c, int max_seq_len, const RecentGeom& rc, int window, bool generic) {
  DecodePlan pl;
  const bool stream_kernel = !generic && stream_ok(c, rc);
  // a sliding window bounds each sequence's range: the window rounded out to
  // whole blocks
  if (window > 0 && max_seq_len > window + kBlock - 1) max_seq_len = window + kBlock - 1;
  // with a recent window the streaming kernel's INT8 splits cover at most
  // max_seq_len - W tokens (the ring goes to the last split's workgroup); the
  // generic kernel's splits cover ring rows too
  const int ring = rc.window > 0 && stream_kernel ? 1 : 0;
  if (ring) max_seq_len = max_seq_len > rc.window ? max_seq_len - rc.window : 1;
  const int gqa = c.num_heads / c.num_kv_heads;
  pl.heads_per_wg = heads_per_wg(gqa);
  const int forced_hpw = env_int("KVQ_HEADS_PER_WG", 0);  // (tests and sweeps)
  if (forced_hpw == 1 || forced_hpw == 2 || forced_hpw == 4)
    if (gqa % forced_hpw == 0) pl.heads_per_wg = forced_hpw;
  const int step = pass_tokens(c.head_dim, stream_kernel);
  // Aim at about one workgroup per compute unit (one round), in whole
  // workgroup passes.  When one round would need splits longer than 2048
  // tokens (large batches of long windows), take about two rounds of the
  // longest length instead (a ragged batch then runs in fewer), with splits
  // of at most 32768 tokens: each workgroup spends about 8 us filling its
  // pipeline, combining its waves and merging its splits, which long splits
  // amortise, and the workgroups run longest sequence first, so the short
  // ones fill the end of the launch.  (On the paged workload, 64 sequences
  // of U[512, 32768] tokens: splits of 32768 tokens 386 us, of 16384 from
  // aiming at four rounds 457 us, of 4096 506 us.)
  const int forced_splits = env_int("KVQ_NUM_SPLITS", 0);
  const int forced_len = env_int("KVQ_SPLIT_LEN", 0);
  int64_t groups = 0;
  int split = 0;
  for (;;) {
    groups = static_cast<int64_t>(c.batch) * c.num_kv_heads * (gqa / pl.heads_per_wg);
    int64_t want = (static_cast<int64_t>(max_seq_len) * groups + kCUs - 1) / kCUs;
    if (want > 2048) {  // several rounds
      want = (static_cast<int64_t>(max_seq_len) * groups + 2 * kCUs - 1) / (2 * kCUs);
      want = want < 2048 ? 2048 : (want > 32768 ? 32768 : want);
    }
    want = want < 512 ? 512 : want;
    split = static_cast<int>(want);
    if (forced_splits > 0) split = (max_seq_len + forced_splits - 1) / forced_splits;
    else if (forced_len > 0) split = forced_len;
    split = ((split + step - 1) / step) * step;
    if (split < step) split = step;
    pl.split_len = split;
    pl.num_splits = split_count(max_seq_len, split);
    if (pl.num_splits < 1) pl.num_splits = 1;
    // A one-round plan that leaves half the compute units idle or more
    // (short contexts, sliding windows) takes fewer heads per workgroup: a
    // KV head's rows are then read by two workgroups, which share its XCD and
    // L2 when the KV heads are a multiple of 8 (consecutive workgroup ids go
    // to consecutive XCDs; otherwise each L2 would fetch the rows again).
    // Sliding decode, 16 sequences x 8 KV heads over a 1024-token window:
    // 15.7 -> 13.5 us.
    if (forced_hpw != 0 || pl.heads_per_wg == 1 || c.num_kv_heads % 8 != 0 || groups * pl.num_splits > kCUs / 2)
      break;
    pl.heads_per_wg /= 2;
  }

  // Longest sequence first pays when workgroups are long (several rounds of
  // splits of 4096 tokens or more): ranking the lengths costs each workgroup
  // a read of the batch's lengths and about batch compare steps up front.
  pl.longest_first = stream_kernel && c.batch > 1 && c.batch <= kLongestFirstMax && split >= 4096;
  const int forced_lf = env_int("KVQ_LONGEST_FIRST", -1);
  if (forced_lf >= 0) pl.longest_first = forced_lf != 0 && stream_kernel && c.batch <= kLongestFirstMax;
  const size_t partials = static_cast<size_t>(c.batch) * c.num_heads * pl.num_splits;
  // per (sequence, head group): the splits' merge-ticket counter
  pl.counter_bytes = align_up(static_cast<size_t>(groups) * sizeof(int32_t), 256);
  pl.workspace = pl.counter_bytes + align_up(partials * 2 * sizeof(float), 256) +
                 partials * static_cast<size_t>(c.head_dim) * sizeof(float);
  return pl;
}

kvq_status launch_decode(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q,
                         const int32_t* seq_lens, float attn_scale, uint16_t* out, void* ws,
                         int max_seq_len, hipStream_t stream, const void* new_k, const void* new_v,
                         int new_dtype, const RecentGeom& rc, int window) {
  const bool append = new_k != nullptr;
  const bool stream_kernel = stream_ok(c, rc);
  // per-head block scales run the streaming kernel, whose fused step
  // quantizes a whole block when its first row leaves the window
  const bool fuse = append && stream_kernel;
  if (append && !fuse) {
    // the generic kernel has no fused path: append the row first
    kvq_status st = launch_append(c, new_k, new_v, new_dtype, 1, seq_lens, stream, true, rc);
    if (st != KVQ_OK) return st;
  }
  DecodeParams p{};  // (chunk mode off)
  p.k_codes = c.k_codes;
  p.v_codes = c.v_codes;
  p.k_scales = c.k_scales;
  p.v_scales = c.v_scales;
  p.scale_bf16 = c.scale_mode == KVQ_SCALE_PER_TOKEN_BF16 ? 1 : 0;
  p.q = q;
  p.seq_lens = seq_lens;
  const size_t partials = static_cast<size_t>(c.batch) * c.num_heads * plan.num_splits;
  char* w = static_cast<char*>(ws);
  p.counters = reinterpret_cast<int32_t*>(w);
  p.part_ml = reinterpret_cast<float*>(w + plan.counter_bytes);
  p.part_o = reinterpret_cast<float*>(w + plan.counter_bytes + align_up(partials * 2 * sizeof(float), 256));
  p.out = out;
  p.new_k = new_k;
  p.new_v = new_v;
  p.new_bf16 = new_dtype == KVQ_DT_BF16 ? 1 : 0;
  p.geom = geom_of(c);
  p.num_heads = c.num_heads;
  p.groups = scales_per_row(c);
  p.split_len = plan.split_len;
  p.num_splits = plan.num_splits;
  const int cap = capacity_of(c);
  p.len_cap = max_seq_len < cap ? max_seq_len : cap;
  const int gqa = c.num_heads / c.num_kv_heads;
  p.wg_per_kvh = gqa / plan.heads_per_wg;
  p.longest_first = plan.longest_first && stream_kernel ? 1 : 0;
  p.balance = plan.split_len >= kBalanceSplit ? 1 : 0;
  p.rk = rc.k;
  p.rv = rc.v;
  p.rwin = rc.window;
  p.rcap = rc.cap;
  p.window = window;
  p.scale_log2 = attn_scale * kLog2e;
  dim3 grid(c.num_kv_heads * p.wg_per_kvh, plan.num_splits, c.batch);
  if (grid.y > 65535 || grid.z > 65535)
    return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_decode: grid too large");
  const int sm = kernel_scale_mode(c);
  const bool paged = c.layout == KVQ_LAYOUT_PAGED;
  p.block_head = fuse && c.scale_mode == KVQ_SCALE_BLOCK_HEAD ? 1 : 0;
  launch_decode_kernel(c.head_dim, stream_kernel, fuse, plan.heads_per_wg, sm, paged, p, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_decode: launch failed: %s", hipGetErrorString(e));
  if (!stream_kernel) {
    hipLaunchKernelGGL(decode_merge_kernel, dim3(c.num_heads, c.batch), dim3(c.head_dim < 256 ? c.head_dim : 256),
                       0, stream, p, c.head_dim);
    e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KVQ_ERR_HIP, "kvq_attention_decode: merge launch failed: %s", hipGetErrorString(e));
  }
  return KVQ_OK;
}

// ---------------------------------------------------------------------------
// Chunked prefill through the generic kernel, for head sizes the MFMA chunk
// kernel does not take: each (sequence, query) pair is one grid row, a decode
// over the keys that query sees (bottom-right causal, optionally a sliding
// window), with its own split partials and merge.
// ---------------------------------------------------------------------------
namespace {

kvq_cache rows_as_batch(const kvq_cache& c, int n) {
  kvq_cache cv = c;
  cv.batch = c.batch * n;
  return cv;
}

}  // namespace

// every supported head dim without an MFMA chunk kernel
bool chunk_generic_supported(int head_dim) { return decode_supported(head_dim) && !chunk_supported(head_dim); }

DecodePlan plan_chunk_generic(const kvq_cache& c, int max_total_len, int n, int window) {
  return plan_decode(rows_as_batch(c, n), max_total_len, RecentGeom(), window, true);
}

kvq_status launch_chunk_generic(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q, int n,
                                const int32_t* ctx_lens, int causal, float attn_scale, uint16_t* out, void* ws,
                                int max_total_len, hipStream_t stream, int window, const RecentGeom& rc) {
  const int64_t rows = static_cast<int64_t>(c.batch) * n;
  if (rows > 65535) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_chunk: batch * n too large (%lld)",
                                static_cast<long long>(rows));
  DecodeParams p{};
  p.k_codes = c.k_codes;
  p.v_codes = c.v_codes;
  p.k_scales = c.k_scales;
  p.v_scales = c.v_scales;
  p.scale_bf16 = c.scale_mode == KVQ_SCALE_PER_TOKEN_BF16 ? 1 : 0;
  p.q = q;
  const size_t partials = static_cast<size_t>(c.batch) * n * c.num_heads * plan.num_splits;
  char* w = static_cast<char*>(ws);
  p.counters = reinterpret_cast<int32_t*>(w);
  p.part_ml = reinterpret_cast<float*>(w + plan.counter_bytes);
  p.part_o = reinterpret_cast<float*>(w + plan.counter_bytes + align_up(partials * 2 * sizeof(float), 256));
  p.out = out;
  p.geom = geom_of(c);
  p.num_heads = c.num_heads;
  p.groups = scales_per_row(c);
  p.split_len = plan.split_len;
  p.num_splits = plan.num_splits;
  const int cap = capacity_of(c);
  p.len_cap = max_total_len < cap ? max_total_len : cap;
  p.wg_per_kvh = (c.num_heads / c.num_kv_heads) / plan.heads_per_wg;
  p.window = window;
  p.scale_log2 = attn_scale * kLog2e;
  p.chunk_n = n;
  p.chunk_causal = causal || window > 0 ? 1 : 0;
  p.ctx_lens = ctx_lens;
  p.rk = rc.k;
  p.rv = rc.v;
  p.rwin = rc.window;
  p.rcap = rc.cap;
  const dim3 grid(c.num_kv_heads * p.wg_per_kvh, plan.num_splits, static_cast<unsigned>(rows));
  if (grid.y > 65535) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_chunk: grid too large");
  const bool paged = c.layout == KVQ_LAYOUT_PAGED;
  launch_generic_any(c.head_dim, plan.heads_per_wg, kernel_scale_mode(c), paged, p, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_chunk: launch failed: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(decode_merge_kernel, dim3(c.num_heads, static_cast<unsigned>(rows)),
                     dim3(c.head_dim < 256 ? c.head_dim : 256), 0, stream, p, c.head_dim);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_chunk: merge launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq
