// Split-K decode attention directly on the INT8 cache.
//
// The method (abaddon 0.2.0-rc.1 src/kv_cache_quant_cuda.rs, module doc:
// fused approach; combs-models 0.2.2 src/kv.rs, `attend`) computes, per query
// head h of KV group g = h / (H/KVH):
//     S_t = scale * sum_d q_d (cK_td - 128) sK_t(d)
//     o   = sum_t softmax(S)_t (cV_td - 128) sV_t(d)
// Design for gfx950:
//   * one workgroup per (sequence, KV head, token split): its 4 waves stream
//     the split's K and V rows once with 16-byte loads, and every byte feeds
//     all query heads of the GQA group handled by the workgroup;
//   * a token row of D bytes is spread over D/16 lanes; codes become floats
//     in registers; the -128 offset is folded out of the inner loop
//     (sum q (c-128) = sum q c - 128 sum q) and per-row scales multiply the
//     partial dot, so no dequantized tile is ever materialised;
//   * softmax is online per lane with a lazy rescale (only when a score
//     exceeds the running max by more than 2^8 in probability);
//   * each split writes (m, l, o) partials; a second kernel merges splits
//     with the log-sum-exp identity and rounds to bf16.
#include "kvq_internal.hpp"

#include <cmath>
#include <cstdlib>

namespace kvq {
namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;      // log2 headroom before a rescale

struct DecodeParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_scales;
  const float* v_scales;
  const uint16_t* q;         // [B, H, D] bf16
  const int32_t* seq_lens;   // [B]
  float* part_o;             // [B, H, S, D]
  float* part_ml;            // [B, H, S, 2]
  uint16_t* out;             // [B, H, D] bf16
  CacheGeom geom;
  int32_t num_heads;
  int32_t groups;            // scales per row
  int32_t split_len;
  int32_t num_splits;
  int32_t len_cap;           // min(hint, capacity)
  int32_t wg_per_kvh;        // workgroups sharing one KV head (GQA group / HPW)
  float scale_log2;          // attn_scale * log2(e)
};

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float byte_f32(uint32_t w, int e) {
  return static_cast<float>((w >> (8 * e)) & 0xffu);  // v_cvt_f32_ubyteN
}

template <int D, int HPW, bool G32>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  constexpr int LPT = D / 16;          // lanes per token row (16 bytes each)
  constexpr int TPW = kWave / LPT;     // token rows per wave pass
  constexpr int TPP = TPW * kWaves;    // token rows per workgroup pass
  constexpr int U = 4;                 // passes issued together

  __shared__ float sm_o[kWaves][HPW][D];
  __shared__ float sm_m[kWaves][HPW];
  __shared__ float sm_l[kWaves][HPW];

  const int split = blockIdx.x;
  const int hg = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = hg / p.wg_per_kvh;
  const int H = p.num_heads;
  const int h0 = kvh * (H / p.geom.kvh) + (hg % p.wg_per_kvh) * HPW;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPT;
  const int slot = lane / LPT;

  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
  const int t_begin = split * p.split_len;
  if (t_begin >= L) return;  // the merge reads only ceil(L / split_len) splits
  const int t_end = min(L, t_begin + p.split_len);
  const int npass = (t_end - t_begin + TPP - 1) / TPP;

  // Query slice of this lane: 16 consecutive dims per head, as fp32.
  float q[HPW][16];
  float qsum[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + (static_cast<int64_t>(b) * H + h0 + j) * D + sub * 16);
    bf16x8_to_f32(qp[0], &q[j][0]);
    bf16x8_to_f32(qp[1], &q[j][8]);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += q[j][e];
    qsum[j] = s;
  }
  const int grp = G32 ? (sub * 16) / 32 : 0;  // scale group of this lane's slice

  float m[HPW], l[HPW], ws[HPW], o[HPW][16];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    ws[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.0f;
  }

  for (int ip = 0; ip < npass; ip += U) {
    uint4 kb[U], vb[U];
    float ks[U], vs[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t_begin + (ip + u) * TPP + wave * TPW + slot;
      int64_t row = -1;
      if (ip + u < npass && t < t_end) row = cache_row(p.geom, b, kvh, t);
      ok[u] = row >= 0;
      if (ok[u]) {
        kb[u] = *reinterpret_cast<const uint4*>(p.k_codes + row * D + sub * 16);
        vb[u] = *reinterpret_cast<const uint4*>(p.v_codes + row * D + sub * 16);
        ks[u] = p.k_scales[row * p.groups + grp];
        vs[u] = p.v_scales[row * p.groups + grp];
      } else {
        kb[u] = make_uint4(0, 0, 0, 0);
        vb[u] = make_uint4(0, 0, 0, 0);
        ks[u] = 0.0f;
        vs[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[4] = {kb[u].x, kb[u].y, kb[u].z, kb[u].w};
      const uint32_t vw[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
      float part[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) part[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = byte_f32(kw[i], e);
#pragma unroll
          for (int j = 0; j < HPW; ++j) part[j] = fmaf(q[j][4 * i + e], c, part[j]);
        }
      }
      float cv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) cv[4 * i + e] = byte_f32(vw[i], e);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float sc = (part[j] - 128.0f * qsum[j]) * ks[u];
        sc = group_sum<LPT>(sc) * p.scale_log2;
        const float sj = ok[u] ? sc : -INFINITY;
        if (sj > m[j] + kLazy) {  // rare: raise the running max
          const float alpha = exp2f(m[j] - sj);
          l[j] *= alpha;
          ws[j] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
          m[j] = sj;
        }
        const float pj = ok[u] ? exp2f(sj - m[j]) : 0.0f;
        l[j] += pj;
        const float w = pj * vs[u];
        ws[j] += w;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = fmaf(w, cv[e], o[j][e]);
      }
    }
  }

  // Fold the +128 offset back in, then combine the token slots of the wave.
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = fmaf(-128.0f, ws[j], o[j][e]);
    float M = m[j];
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) M = fmaxf(M, shfl_xor_f32(M, off));
    const float f = (m[j] == -INFINITY) ? 0.0f : exp2f(m[j] - M);
    l[j] *= f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] *= f;
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
      l[j] += shfl_xor_f32(l[j], off);
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j][e] += shfl_xor_f32(o[j][e], off);
    }
    m[j] = M;
  }
  if (slot == 0) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sm_o[wave][j][sub * 16 + e] = o[j][e];
      if (sub == 0) {
        sm_m[wave][j] = m[j];
        sm_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HPW * D; idx += kThreads) {
    const int j = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = sm_m[w][j] == -INFINITY ? 0.0f : exp2f(sm_m[w][j] - M);
      acc = fmaf(sm_o[w][j][d], f, acc);
      lsum = fmaf(sm_l[w][j], f, lsum);
    }
    const int64_t pidx = (static_cast<int64_t>(b) * H + h0 + j) * p.num_splits + split;
    p.part_o[pidx * D + d] = acc;
    if (d == 0) {
      p.part_ml[pidx * 2] = M;
      p.part_ml[pidx * 2 + 1] = lsum;
    }
  }
}

// Log-sum-exp merge of the split partials of one (sequence, head); bf16 out.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int D) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int H = p.num_heads;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
  const int ns = (L + p.split_len - 1) / p.split_len;
  const int64_t base = (static_cast<int64_t>(b) * H + h) * p.num_splits;
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
    }
    const float v = den > 0.0f ? num / den : 0.0f;
    p.out[(static_cast<int64_t>(b) * H + h) * D + d] = f32_to_bf16_rne(v);
  }
}

int heads_per_wg(int gqa) {
  if (gqa % 4 == 0) return 4;
  if (gqa % 2 == 0) return 2;
  return 1;
}

int lanes_per_token(int D) { return D / 16; }

template <int D, int HPW>
void launch_split(const DecodeParams& p, bool g32, dim3 grid, hipStream_t st) {
  if (g32)
    hipLaunchKernelGGL((decode_split_kernel<D, HPW, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, HPW, false>), grid, dim3(kThreads), 0, st, p);
}

template <int D>
void launch_split_d(const DecodeParams& p, int hpw, bool g32, dim3 grid, hipStream_t st) {
  if (hpw == 4) launch_split<D, 4>(p, g32, grid, st);
  else if (hpw == 2) launch_split<D, 2>(p, g32, grid, st);
  else launch_split<D, 1>(p, g32, grid, st);
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

}  // namespace

bool decode_supported(int head_dim) {
  return head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256;
}

DecodePlan plan_decode(const kvq_cache& c, int max_seq_len) {
  DecodePlan pl;
  const int gqa = c.num_heads / c.num_kv_heads;
  pl.heads_per_wg = heads_per_wg(gqa);
  const int tpp = (kWave / lanes_per_token(c.head_dim)) * kWaves;
  int split = 512;
  const int forced_splits = env_int("KVQ_NUM_SPLITS", 0);
  const int forced_len = env_int("KVQ_SPLIT_LEN", 0);
  if (forced_splits > 0) split = (max_seq_len + forced_splits - 1) / forced_splits;
  else if (forced_len > 0) split = forced_len;
  split = ((split + tpp - 1) / tpp) * tpp;
  if (split < tpp) split = tpp;
  pl.split_len = split;
  pl.num_splits = (max_seq_len + split - 1) / split;
  if (pl.num_splits < 1) pl.num_splits = 1;
  pl.workspace = static_cast<size_t>(c.batch) * c.num_heads * pl.num_splits *
                 (static_cast<size_t>(c.head_dim) + 2) * sizeof(float);
  return pl;
}

kvq_status launch_decode(const kvq_cache& c, const DecodePlan& plan, const uint16_t* q,
                         const int32_t* seq_lens, float attn_scale, uint16_t* out, void* ws,
                         int max_seq_len, hipStream_t stream) {
  DecodeParams p;
  p.k_codes = c.k_codes;
  p.v_codes = c.v_codes;
  p.k_scales = c.k_scales;
  p.v_scales = c.v_scales;
  p.q = q;
  p.seq_lens = seq_lens;
  p.part_o = static_cast<float*>(ws);
  p.part_ml = p.part_o + static_cast<size_t>(c.batch) * c.num_heads * plan.num_splits * c.head_dim;
  p.out = out;
  p.geom = geom_of(c);
  p.num_heads = c.num_heads;
  p.groups = scales_per_row(c);
  p.split_len = plan.split_len;
  p.num_splits = plan.num_splits;
  const int cap = capacity_of(c);
  p.len_cap = max_seq_len < cap ? max_seq_len : cap;
  const int gqa = c.num_heads / c.num_kv_heads;
  p.wg_per_kvh = gqa / plan.heads_per_wg;
  p.scale_log2 = attn_scale * kLog2e;
  dim3 grid(plan.num_splits, c.num_kv_heads * p.wg_per_kvh, c.batch);
  if (grid.y > 65535 || grid.z > 65535)
    return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_decode: grid too large");
  const bool g32 = c.scale_mode == KVQ_SCALE_GROUP32;
  switch (c.head_dim) {
    case 32: launch_split_d<32>(p, plan.heads_per_wg, g32, grid, stream); break;
    case 64: launch_split_d<64>(p, plan.heads_per_wg, g32, grid, stream); break;
    case 128: launch_split_d<128>(p, plan.heads_per_wg, g32, grid, stream); break;
    default: launch_split_d<256>(p, plan.heads_per_wg, g32, grid, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_decode: split launch failed: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(decode_merge_kernel, dim3(c.num_heads, c.batch), dim3(c.head_dim < 256 ? c.head_dim : 256), 0,
                     stream, p, c.head_dim);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_decode: merge launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq
