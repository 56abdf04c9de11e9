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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Ring rows of a chunk on a hybrid cache, after the MFMA chunk kernel has
// attended to the INT8 keys.  The queries that see ring rows are the last
// min(n, W) of each sequence (ctx_lens clamped to the hint); the others
// already have their output.  One workgroup per (sequence, group of HPW
// query heads, four of those queries), one wave per query: the ring rows the
// four see are staged in LDS 64 at a time, then each wave runs LPT lanes per
// row with the same per-lane online softmax as the generic kernel, folds in
// the MFMA kernel's partial (m, l, o) for its query and writes the
// normalised row as bf16.
template <int D, int HPW>
__global__ __launch_bounds__(256) void chunk_ring_kernel(DecodeParams p) {
  constexpr int LPT = D / 16;
  constexpr int TPW = kWave / LPT;
  constexpr int kQPB = 256 / kWave;       // queries per workgroup
  constexpr int kTile = 64;               // ring rows staged per step
  constexpr int kRow = 2 * D + 16;        // LDS row bytes (padded)
  constexpr int kPer = kTile * (D / 8) / 256;  // 16-byte pieces per thread and side
  __shared__ __attribute__((aligned(16))) uint8_t sk[kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t sv[kTile * kRow];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int groups = p.geom.kvh * p.wg_per_kvh;
  const int nq = p.chunk_n;
  const int nt = nq - p.chunk_q0;  // ring-seeing queries per sequence
  const int qblocks = (nt + kQPB - 1) / kQPB;
  const int hg = blockIdx.x % groups;
  // the last queries see the most ring rows: their workgroups go first
  const int qb = qblocks - 1 - (blockIdx.x / groups) % qblocks;
  const int b = blockIdx.x / groups / qblocks;
  const int r = qb * kQPB + wave;         // this wave's partial row in the sequence
  const bool active = r < nt;
  const int qi = p.chunk_q0 + min(r, nt - 1);
  const int L0 = min(max(p.ctx_lens[b], 0), p.len_cap - nq);
  const int L = L0 + qi + 1;                  // keys this query sees
  const int L8 = max(L0 + nq - p.rwin, 0);    // first ring row (L > L8)
  const int Lblk = L0 + p.chunk_q0 + min(qb * kQPB + kQPB, nt);  // keys the workgroup's last query sees
  const int kvh = hg / p.wg_per_kvh;
  const int H = p.num_heads;
  const int h0 = kvh * (H / p.geom.kvh) + (hg % p.wg_per_kvh) * HPW;
  const int sub = lane % LPT;
  const int slot = lane / LPT;
  const int64_t v = static_cast<int64_t>(b) * nt + min(r, nt - 1);  // partial row

  // queries and ring K stay bf16 pairs: scores use v_dot2_f32_bf16 (exact
  // products, fp32 sums)
  uint32_t q[HPW][8];
  float pm[HPW], pl[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const uint4* qp =
        reinterpret_cast<const uint4*>(p.q + ((static_cast<int64_t>(b) * H + h0 + j) * nq + qi) * D + sub * 16);
    const uint4 q0 = qp[0], q1 = qp[1];
    q[j][0] = q0.x; q[j][1] = q0.y; q[j][2] = q0.z; q[j][3] = q0.w;
    q[j][4] = q1.x; q[j][5] = q1.y; q[j][6] = q1.z; q[j][7] = q1.w;
    pm[j] = p.part_ml[(v * H + h0 + j) * 2];
    pl[j] = p.part_ml[(v * H + h0 + j) * 2 + 1];
  }
  float m[HPW], l[HPW], o[HPW][16];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.0f;
  }

  const int64_t ring0 = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.rcap;
  for (int t0 = L8; t0 < Lblk; t0 += kTile) {  // (block-uniform bounds: every wave meets the barriers)
    const int nrows = min(kTile, Lblk - t0);
    uint4 kr[kPer], vr[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = threadIdx.x + i * 256;
      const int64_t row = ring0 + (t0 + min(id / (D / 8), nrows - 1)) % p.rcap;
      kr[i] = *reinterpret_cast<const uint4*>(p.rk + row * D + (id % (D / 8)) * 8);
      vr[i] = *reinterpret_cast<const uint4*>(p.rv + row * D + (id % (D / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = threadIdx.x + i * 256;
      *reinterpret_cast<uint4*>(sk + (id / (D / 8)) * kRow + (id % (D / 8)) * 16) = kr[i];
      *reinterpret_cast<uint4*>(sv + (id / (D / 8)) * kRow + (id % (D / 8)) * 16) = vr[i];
    }
    __syncthreads();
    const int tend = active ? min(t0 + kTile, L) : t0;
    for (int tb = t0; tb < tend; tb += TPW) {
      const int t = tb + slot;
      const bool ok = t < tend;
      const int rr = min(t, tend - 1) - t0;
      const uint4* kp = reinterpret_cast<const uint4*>(sk + rr * kRow + sub * 32);
      const uint4* vp = reinterpret_cast<const uint4*>(sv + rr * kRow + sub * 32);
      const uint4 k0 = kp[0], k1 = kp[1];
      const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      float vx[16];
      bf16x8_to_f32(vp[0], &vx[0]);
      bf16x8_to_f32(vp[1], &vx[8]);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float pa = 0.0f, pb = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          pa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[j][e]), __builtin_bit_cast(bf16x2, kw[e]), pa,
                                               false);
          pb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[j][e + 1]),
                                               __builtin_bit_cast(bf16x2, kw[e + 1]), pb, false);
        }
        const float sc = group_sum<LPT>(pa + pb) * p.scale_log2;
        const float sj = ok ? sc : -INFINITY;
        if (sj > m[j] + kLazy) {  // lazy running maximum: weights stay below 2^8
          const float alpha = __builtin_amdgcn_exp2f(m[j] - sj);  // 0 on the first key (m = -inf)
          l[j] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
          m[j] = sj;
        }
        const float pj = ok ? __builtin_amdgcn_exp2f(sj - m[j]) : 0.0f;
        l[j] += pj;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = fmaf(pj, vx[e], o[j][e]);
      }
    }
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    // combine the lane slots (every query here sees a ring row, so M is finite)
    const float M = slot_max<LPT>(m[j]);
    const float f = m[j] == -INFINITY ? 0.0f : exp2f(m[j] - M);
    const float lj = slot_sum<LPT>(l[j] * f);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = slot_sum<LPT>(o[j][e] * f);
    // fold in the INT8 keys' partial
    const float M2 = fmaxf(M, pm[j]);
    const float fa = exp2f(M - M2);
    const float fb = pm[j] == -INFINITY ? 0.0f : exp2f(pm[j] - M2);
    const float inv = 1.0f / fmaf(lj, fa, pl[j] * fb);
    if (slot == 0) {
      float* po = p.part_o + (v * H + h0 + j) * D + sub * 16;
      uint16_t* orow = p.out + ((static_cast<int64_t>(b) * H + h0 + j) * nq + qi) * D + sub * 16;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const float4 pv = *reinterpret_cast<const float4*>(po + e);
        ushort4 w;
        w.x = f32_to_bf16_rne(fmaf(o[j][e + 0], fa, pv.x * fb) * inv);
        w.y = f32_to_bf16_rne(fmaf(o[j][e + 1], fa, pv.y * fb) * inv);
        w.z = f32_to_bf16_rne(fmaf(o[j][e + 2], fa, pv.z * fb) * inv);
        w.w = f32_to_bf16_rne(fmaf(o[j][e + 3], fa, pv.w * fb) * inv);
        *reinterpret_cast<ushort4*>(orow + e) = w;
        // the workspace goes back to zero (this wave alone reads the row)
        *reinterpret_cast<float4*>(po + e) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
      if (sub == 0) {
        p.part_ml[(v * H + h0 + j) * 2] = 0.0f;
        p.part_ml[(v * H + h0 + j) * 2 + 1] = 0.0f;
      }
    }
  }
}

int heads_per_wg(int gqa) {
  if (gqa % 4 == 0) return 4;
  if (gqa % 2 == 0) return 2;
  return 1;
}

bool use_stream(int head_dim) { return head_dim == 32 || head_dim == 64 || head_dim == 128; }

// The streaming kernel takes head dims 32, 64 and 128 in every per-row scale
// mode; per-channel block scales run on the generic kernel.
bool stream_ok(const kvq_cache& c) { return use_stream(c.head_dim) && c.scale_mode != KVQ_SCALE_BLOCK_CHANNEL; }

int pass_tokens(int head_dim, bool stream_kernel) {
  // tokens a workgroup consumes per step: whole 64-token wave blocks for the
  // streaming kernel, one pass of all waves for the generic kernel
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
  const bool stream_kernel = !generic && stream_ok(c);
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
  // tokens (large batches of long windows), take about four rounds instead,
  // with splits of at most 16384 tokens: each workgroup spends a fixed few
  // microseconds filling its pipeline and combining its waves, which long
  // splits amortise, while ragged batches stay balanced across rounds.
  const int64_t groups = static_cast<int64_t>(c.batch) * c.num_kv_heads * (gqa / pl.heads_per_wg);
  int64_t want = (static_cast<int64_t>(max_seq_len) * groups + kCUs - 1) / kCUs;
  if (want > 2048) {  // several rounds
    want = (static_cast<int64_t>(max_seq_len) * groups + 4 * kCUs - 1) / (4 * kCUs);
    want = want < 2048 ? 2048 : (want > 16384 ? 16384 : want);
  }
  want = want < 512 ? 512 : want;
  int split = static_cast<int>(want);
  const int forced_splits = env_int("KVQ_NUM_SPLITS", 0);
  const int forced_len = env_int("KVQ_SPLIT_LEN", 0);
  if (forced_splits > 0) split = (max_seq_len + forced_splits - 1) / forced_splits;
  else if (forced_len > 0) split = forced_len;
  split = ((split + step - 1) / step) * step;
  if (split < step) split = step;
  pl.split_len = split;
  pl.num_splits = split_count(max_seq_len, split);
  if (pl.num_splits < 1) pl.num_splits = 1;

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
  const bool stream_kernel = stream_ok(c);
  if (append && (!stream_kernel || is_block_mode(c))) {
    // the generic kernel has no fused path, and a block-scale step may
    // quantize a whole block: append the row first
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
  const bool fused = append && stream_kernel && !is_block_mode(c);
  launch_decode_kernel(c.head_dim, stream_kernel, fused, plan.heads_per_wg, sm, paged, p, grid, stream);
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

DecodePlan plan_chunk_hybrid(const kvq_cache& c, int n, int recent_window) {
  // one partial (the INT8 keys') per (sequence, ring-seeing query, head)
  DecodePlan pl{};
  pl.heads_per_wg = heads_per_wg(c.num_heads / c.num_kv_heads);
  pl.num_splits = 1;
  pl.counter_bytes = 0;
  const size_t partials = static_cast<size_t>(c.batch) * (n < recent_window ? n : recent_window) * c.num_heads;
  pl.workspace = align_up(partials * 2 * sizeof(float), 256) + partials * static_cast<size_t>(c.head_dim) * sizeof(float);
  return pl;
}

kvq_status launch_chunk_generic(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q, int n,
                                const int32_t* ctx_lens, int causal, float attn_scale, uint16_t* out, void* ws,
                                int max_total_len, hipStream_t stream, int window, const RecentGeom& rc,
                                bool int8_on_mfma) {
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
  const int nt = int8_on_mfma ? (n < rc.window ? n : rc.window) : n;  // hybrid: partial rows per sequence
  const size_t partials = static_cast<size_t>(c.batch) * nt * c.num_heads * plan.num_splits;
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
  if (int8_on_mfma) {
    // the MFMA chunk kernel attends to the INT8 keys (partials for the
    // queries that also see ring rows), then one wave per (row, head group)
    // takes the ring rows and writes those queries' outputs
    ChunkPartials cp;
    cp.rwin = rc.window;
    cp.stride = 1;
    cp.slot = 0;
    cp.o = p.part_o;
    cp.ml = p.part_ml;
    const kvq_status st = launch_chunk(c, q, n, ctx_lens, 1, attn_scale, out, ws, max_total_len - n, stream, 0, &cp);
    if (st != KVQ_OK) return st;
    p.chunk_q0 = n - nt;
    p.batch_rows = c.batch;
    // one workgroup per (sequence, four ring-seeing queries, head group)
    const int64_t blocks = static_cast<int64_t>(c.batch) * ((nt + 3) / 4) * c.num_kv_heads * p.wg_per_kvh;
    if (blocks > 0x7fffffffLL) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_chunk_recent: grid too large");
    const dim3 rgrid(static_cast<unsigned>(blocks));
    const int hpw = plan.heads_per_wg;
    if (c.head_dim == 128) {
      if (hpw == 4) hipLaunchKernelGGL((chunk_ring_kernel<128, 4>), rgrid, dim3(256), 0, stream, p);
      else if (hpw == 2) hipLaunchKernelGGL((chunk_ring_kernel<128, 2>), rgrid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((chunk_ring_kernel<128, 1>), rgrid, dim3(256), 0, stream, p);
    } else {
      if (hpw == 4) hipLaunchKernelGGL((chunk_ring_kernel<64, 4>), rgrid, dim3(256), 0, stream, p);
      else if (hpw == 2) hipLaunchKernelGGL((chunk_ring_kernel<64, 2>), rgrid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((chunk_ring_kernel<64, 1>), rgrid, dim3(256), 0, stream, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KVQ_ERR_HIP, "kvq_attention_chunk_recent: ring launch failed: %s", hipGetErrorString(e));
    return KVQ_OK;
  }
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
