// Streaming decode kernel and the device helpers it shares with the
// generic kernel, split-merge and recent-window ring code.  Included by
// kvq_decode.hip (INT8 scale modes, the generic kernel, the planner and
// the launch) and kvq_decode_fp8.hip (FP8 codes), so the kernel
// instantiations compile in two translation units.
//
// Split-K decode attention directly on the INT8 cache.
//
// The method (abaddon 0.2.0-rc.1 src/kv_cache_quant_cuda.rs, module doc:
// fused approach; combs-models 0.2.2 src/kv.rs, `attend`) computes, per query
// head h of KV group g = h / (H/KVH):
//     S_t = scale * sum_d q_d (cK_td - 128) sK_t(d)
//     o   = sum_t softmax(S)_t (cV_td - 128) sV_t(d)
//
// gfx950 design of the streaming kernel (head_dim 32, 64, 128, 256):
//   * one workgroup = (sequence, KV head (and a share of its query heads),
//     token split); its 8 waves take blocks of 64 tokens (32 at head dim
//     256: 16 KB of K and V either way) in turn.  Every loaded byte serves
//     all the query heads of the workgroup (one K/V read per GQA group).
//   * codes are never widened to fp32: v_perm_b32 places two code bytes into
//     the low bytes of two f16 halves (the f16 values c * 2^-24, exact).  The
//     scores are matrix-core products S = Q K^T of 16-token groups
//     (v_mfma_f32_16x16x32_f16; head dim 32: v_dot2_f32_f16 partial dots
//     summed through LDS), and PV multiplies f16 softmax weights with pairs
//     of tokens' codes in v_dot2_f32_f16, accumulating in fp32.  The -128
//     offset is folded out: sum x (c - 128) = sum x c - 128 sum x.  Queries
//     are scaled by a power of two into [2^14, 2^15) first, which is exact
//     for bf16 inputs.
//   * the softmax of each token is computed once, by one lane; per-token V
//     scales are folded into the exponent (w = 2^(S + log2 sV - m)), so the
//     weights stay in f16 range; the running maximum is wave-uniform and
//     only rescales the accumulators when a score exceeds it by more than
//     2^8.
//   * the next block's K (and V) rows are loaded while the current block is
//     computed;
//   * each split leaves (m, l, o) partials; the split that draws the last
//     ticket of its (sequence, head group) merges them with the log-sum-exp
//     identity and writes bf16.
// Head dim 256 with a recent window, per-channel block scales and head dims
// 96-224 use the generic kernel of kvq_decode.hip (fp32 FMAs, separate merge).
#pragma once

#include "kvq_internal.hpp"
#include "kvq_quant.hpp"

#include <cmath>
#include <cstdlib>
#include <type_traits>

namespace kvq {

struct DecodeParams {
  uint8_t* k_codes;          // written only by the fused append
  uint8_t* v_codes;
  float* k_scales;
  float* v_scales;
  const uint16_t* q;         // [B, H, D] bf16
  const int32_t* seq_lens;   // [B]
  int32_t* counters;         // [B, KVH * wg_per_kvh], zero between calls
  float* part_ml;            // [B, H, S, 2]  (m, l) per split
  float* part_o;             // [B, H, S, D]  unnormalised outputs
  uint16_t* out;             // [B, H, D] bf16
  const void* new_k;         // fused append: K/V rows [B, KVH, 1, D] for position seq_lens[b] - 1
  const void* new_v;
  int32_t new_bf16;          // fused append: rows are bf16 (else fp32)
  CacheGeom geom;
  int32_t num_heads;
  int32_t groups;            // scales per row
  int32_t split_len;
  int32_t num_splits;
  int32_t len_cap;           // min(hint, capacity)
  int32_t wg_per_kvh;        // workgroups sharing one KV head (GQA group / HPW)
  int32_t longest_first;     // workgroup z takes the z-th longest sequence (batch <= kLongestFirstMax)
  int32_t balance;           // paired waves of a SIMD keep pace through their priority (long splits)
  float scale_log2;          // attn_scale * log2(e)
  // recent window (hybrid cache): the last rwin positions are bf16 rows in
  // ring slot (position % rcap), attended by the workgroup of the last INT8 split
  uint16_t* rk;              // [B, KVH, rcap, D] bf16
  uint16_t* rv;
  int32_t rwin, rcap;        // rwin 0: no recent window
  // sliding window (0: none): the query at position L - 1 sees keys in
  // (L - 1 - window, L - 1]
  int32_t window;
  int32_t scale_bf16;        // per-token scales stored as bf16
  // chunked prefill through the generic kernel (chunk_n > 0): grid z runs over
  // (sequence b, query i) pairs, b * chunk_n + i, each a decode over the keys
  // query i sees; q and out are [B, H, chunk_n, D]
  int32_t chunk_n;
  int32_t chunk_causal;      // query i sees keys t <= ctx_lens[b] + i (else all ctx + n)
  const int32_t* ctx_lens;   // [B], tokens cached before the chunk
  // fused append on a hybrid cache with per-head block scales: the step
  // whose leaving row starts a 16-row block quantizes the whole block
  int32_t block_head;
};

namespace {

constexpr int kWaves = 4;          // waves per workgroup (generic kernel)
constexpr int kThreads = kWaves * kWave;
constexpr int kStreamWaves = 8;    // waves per workgroup (streaming kernel): 2 per SIMD
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kCUs = 256;          // MI355X compute units: the split heuristic aims at one workgroup each
constexpr int kBlock = 64;         // tokens per wave block (streaming kernel)
constexpr int kLongestFirstMax = kStreamThreads;  // largest batch ranked by length in a workgroup
constexpr int kBalanceSplit = 4096;  // splits at least this long pace each SIMD's two waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSmToken = KVQ_SCALE_PER_TOKEN;         // scale modes, as kernel template arguments
constexpr int kSmGroup32 = KVQ_SCALE_GROUP32;
constexpr int kSmTokenBf16 = KVQ_SCALE_PER_TOKEN_BF16;
constexpr int kSmFp8E4M3 = KVQ_CODES_FP8_E4M3;          // FP8 codes, no scales
constexpr int kSmFp8E5M2 = KVQ_CODES_FP8_E5M2;
constexpr int kSmBlockChannel = KVQ_SCALE_BLOCK_CHANNEL;  // per-channel block scales (generic kernel)
constexpr float kLazy = 8.0f;      // log2 headroom before a rescale
constexpr int kWeightShift = 7;    // weights carry 2^7 so they fill f16 range

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));


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

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// f16 pair (1024 + c0, 1024 + c1) -> (c0 - 128, c1 - 128), exact.
__device__ __forceinline__ uint32_t exact_pair(uint32_t w) {
  const half2_t off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, w) + off);
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

__device__ __forceinline__ float f16_value(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Loads of K and V codes, which each launch reads once: non-temporal, so
// that the stream does not push out of L2 what is read again (the kernel's
// own code among it: an instruction fetch that misses L2 waits for HBM).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* ptr) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const uint8_t* ptr) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(ptr));
  return make_uint2(v.x, v.y);
}

// Maximum over aligned groups of N consecutive lanes (N in {1,2,4,8,16}).
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}

// {x_i, x_(i^32)} and {x_i, x_(i^16)} for every lane i, without LDS
// (v_permlane32_swap / v_permlane16_swap on the same register).
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  float a, b;
  x = group_max<16>(x);
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum(float x) {
  float a, b;
  x = group_sum<16>(x);
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}

// Sum over the lanes that share (lane % LPT): the token slots of a wave.
template <int LPT>
__device__ __forceinline__ float slot_sum(float x) {
  float a, b;
  if constexpr (LPT <= 1) x += dpp_f32<0x121>(x);  // row_ror:1
  if constexpr (LPT <= 2) x += dpp_f32<0x122>(x);  // row_ror:2
  if constexpr (LPT <= 4) x += dpp_f32<0x124>(x);  // row_ror:4
  if constexpr (LPT <= 8) x += dpp_f32<0x128>(x);  // row_ror:8
  if constexpr (LPT <= 16) {
    swap16(x, a, b);
    x = a + b;
  }
  swap32(x, a, b);
  return a + b;
}

// Maximum over the lanes that share (lane % LPT).
template <int LPT>
__device__ __forceinline__ float slot_max(float x) {
  float a, b;
  if constexpr (LPT <= 1) x = fmaxf(x, dpp_f32<0x121>(x));  // row_ror:1
  if constexpr (LPT <= 2) x = fmaxf(x, dpp_f32<0x122>(x));  // row_ror:2
  if constexpr (LPT <= 4) x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  if constexpr (LPT <= 8) x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
  if constexpr (LPT <= 16) {
    swap16(x, a, b);
    x = fmaxf(a, b);
  }
  swap32(x, a, b);
  return fmaxf(a, b);
}

// Value of lane (i + N) for lanes whose partner lies in the same 32-lane half.
template <int N>
__device__ __forceinline__ uint32_t lane_up(uint32_t x) {
  if constexpr (N < 16) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x100 + N, 0xF, 0xF, false));
  } else {
    static_assert(N == 16, "partner distance");
    return __builtin_amdgcn_permlane16_swap(x, x, false, false)[1];
  }
}

// 2^x with the hardware instruction (results below the normal range flush to
// zero, which only drops weights that could not change a bf16 output).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// True when the condition holds in any lane of the wave (scalar result).
__device__ __forceinline__ bool any_lane(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// A value every lane holds equally, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Orders this wave's LDS writes before its following LDS reads (lanes of one
// wave exchange data through LDS; no other wave takes part).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Splits of a token range of `len` tokens: whole splits of split_len, and a
// remainder of at most one block joins the last one (a split of a few tokens
// would cost a workgroup and a merge input for almost no work).
__host__ __device__ inline int split_count(int len, int split_len) {
  if (len <= 0) return 0;
  const int full = len / split_len;
  if (full == 0) return 1;
  return full + (len - full * split_len > kBlock ? 1 : 0);
}

__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  int L = p.seq_lens[b];
  return L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
}

// The sequence b and query qi of grid row v, and the keys that query sees:
// decode, v = b; chunk mode, v = b * chunk_n + qi.
__device__ __forceinline__ int row_len(const DecodeParams& p, int v, int& b, int& qi) {
  if (p.chunk_n == 0) {
    b = v;
    qi = 0;
    return clamp_len(p, b);
  }
  b = v / p.chunk_n;
  qi = v % p.chunk_n;
  int L0 = p.ctx_lens[b];
  L0 = L0 < 0 ? 0 : (L0 > p.len_cap ? p.len_cap : L0);
  const int L = p.chunk_causal ? L0 + qi + 1 : L0 + p.chunk_n;
  return L > p.len_cap ? p.len_cap : L;
}

// First ring position of a hybrid cache for grid row (b, L) (L itself
// without a recent window): the last rwin of the L decode tokens, or of the
// ctx + chunk_n rows the cache holds in chunk mode.
__device__ __forceinline__ int ring_start(const DecodeParams& p, int b, int L) {
  if (p.rwin <= 0) return L;
  int Lc = L;
  if (p.chunk_n > 0) {
    const int c0 = min(max(p.ctx_lens[b], 0), p.len_cap);
    Lc = min(c0 + p.chunk_n, p.len_cap);
  }
  return max(Lc - p.rwin, 0);
}

// The sequence a workgroup serves.  With longest_first set (batch at most NT),
// workgroup z takes the z-th longest sequence, ties in index order: when the
// grid runs in several rounds the long sequences start first and the ragged
// end of the launch is made of short ones.  Each (sequence, head) result is
// the same whichever workgroup computes it.  `scratch` is NT ints of LDS
// that no wave writes before it has returned from here.  `len` receives the
// sequence's clamped length when the ranking has read it, else -1.
template <int NT>
__device__ __forceinline__ int sequence_of(const DecodeParams& p, int* scratch, int& len) {
  const int z = blockIdx.z;
  len = -1;
  if (!p.longest_first) return z;
  __shared__ int sm_seq;
  const int nb = gridDim.z;
  const int t = threadIdx.x;
  const int lt = t < nb ? clamp_len(p, t) : 0;
  scratch[t] = lt;
  __syncthreads();
  if (t < nb) {
    int r = 0;  // sequences ahead of t
    for (int j = 0; j < nb; ++j) {
      const int lj = scratch[j];
      r += (lj > lt) | ((lj == lt) & (j < t));
    }
    if (r == z) sm_seq = t;  // the ranks are a permutation of 0..nb-1
  }
  __syncthreads();
  const int b = __builtin_amdgcn_readfirstlane(sm_seq);
  len = __builtin_amdgcn_readfirstlane(scratch[b]);
  return b;
}

// ---------------------------------------------------------------------------
// Split partials between workgroups.  A word of the partial area reads zero
// until its split has written it, so the data is its own ready flag: a value
// whose bits are zero (+0.0) is stored as -0.0, which every use treats alike,
// and the merging workgroup returns each word it consumed to zero for the
// next call.  Stores and loads are agent-scope atomics (they bypass the
// per-XCD L2), so a merger on another XCD sees them without an L2 write-back
// or invalidate.
// ---------------------------------------------------------------------------
constexpr int kPollBudget = 1 << 20;  // polling rounds per thread before a missing partial reads as zero

__device__ __forceinline__ void put_partial(float* dst, float x) {
  const uint32_t u = __float_as_uint(x);
  __hip_atomic_store(reinterpret_cast<uint32_t*>(dst), u == 0u ? 0x80000000u : u, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t peek_partial(const float* src) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Words w1[k], w2[k] are first readings of a1[k], a2[k] (a slot not taken
// part in holds a nonzero dummy and is never read).  Every word still reading
// zero (not written yet) is read again, all of them together, until none is,
// within
// the thread's poll budget (which bounds the wait should a writer never
// come; such a word then stays +0.0).
template <int N, int M>
__device__ __forceinline__ void await_partials(float* const (&a1)[N], uint32_t (&w1)[N], float* const (&a2)[M],
                                               uint32_t (&w2)[M], int& budget) {
  for (;;) {
    bool missing = false;
#pragma unroll
    for (int k = 0; k < N; ++k) missing |= w1[k] == 0u;
#pragma unroll
    for (int k = 0; k < M; ++k) missing |= w2[k] == 0u;
    if (!missing || budget <= 0) return;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (w1[k] == 0u) w1[k] = peek_partial(a1[k]);
#pragma unroll
    for (int k = 0; k < M; ++k)
      if (w2[k] == 0u) w2[k] = peek_partial(a2[k]);
    --budget;
  }
}

template <int N>
__device__ __forceinline__ void await_partials(float* const (&a)[N], uint32_t (&w)[N], int& budget) {
  float* const none[1] = {nullptr};
  uint32_t one[1] = {1u};  // (a dummy slot, never read)
  await_partials(a, w, none, one, budget);
}

__device__ __forceinline__ void clear_partial(float* dst) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(dst), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Final output of HPW heads, from the workgroup's own combined partial
// (sm_o, sm_ml) when the sequence has one split, else by the merging
// workgroup.  Every split of a (sequence, head group) takes a ticket from its
// counter once its first wave is through its tokens; the one that draws the
// last ticket merges, and `last` says whether this is it.  Since
// the others drew theirs first they are running and write their partials
// without waiting on anything, so the merger's wait for them always ends.
// The merger keeps its own partial in LDS.
// ---------------------------------------------------------------------------
template <int D, int HPW, int NT>
__device__ void finish_split(const DecodeParams& p, int b, int h0, int split, int ns, bool last,
                             const float (*sm_o)[D], const float (*sm_ml)[2]) {
  const int H = p.num_heads;
  if (ns == 1) {
    for (int idx = threadIdx.x; idx < HPW * D; idx += NT) {
      const int j = idx / D, d = idx % D;
      const float l = sm_ml[j][1];
      const float v = l > 0.0f ? sm_o[j][d] / l : 0.0f;
      p.out[(static_cast<int64_t>(b) * H + h0 + j) * D + d] = f32_to_bf16_rne(v);
    }
    return;
  }
  if (!last) {
    for (int idx = threadIdx.x; idx < HPW * D; idx += NT) {
      const int j = idx / D, d = idx % D;
      const int64_t pidx = (static_cast<int64_t>(b) * H + h0 + j) * p.num_splits + split;
      put_partial(&p.part_o[pidx * D + d], sm_o[j][d]);
      if (d == 0) {
        put_partial(&p.part_ml[pidx * 2], sm_ml[j][0]);
        put_partial(&p.part_ml[pidx * 2 + 1], sm_ml[j][1]);
      }
    }
    return;
  }
  int budget = kPollBudget;

  // Merge in split order (the same order whichever split merges), this
  // split's (m, l, o) from LDS.  A round stages the (m, l) of up to kChunk
  // splits in LDS; the first readings of those and of this thread's o words
  // of the round's first kU splits all go out before anything is waited for.
  constexpr int kChunk = NT / HPW;   // splits whose (m, l) one round stages in LDS
  constexpr int kItems = (HPW * D + NT - 1) / NT;
  constexpr int kU = 8;              // splits whose o words one pass reads
  __shared__ float sm_sm[HPW][kChunk];
  __shared__ float sm_sl[HPW][kChunk];
  float run_m[kItems], num[kItems], den[kItems];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    run_m[it] = -INFINITY;
    num[it] = 0.0f;
    den[it] = 0.0f;
  }
  for (int c0 = 0; c0 < ns; c0 += kChunk) {
    const int cnt_c = min(kChunk, ns - c0);
    const int jm = threadIdx.x / kChunk, um = threadIdx.x % kChunk;
    const bool own_ml = um < cnt_c && c0 + um != split;
    float* mlp = &p.part_ml[((static_cast<int64_t>(b) * H + h0 + jm) * p.num_splits + c0 + min(um, cnt_c - 1)) * 2];
    float* const ma[2] = {mlp, mlp + 1};
    uint32_t mw[2] = {own_ml ? peek_partial(ma[0]) : 1u, own_ml ? peek_partial(ma[1]) : 1u};
    float* oa[kItems][kU];
    uint32_t ow[kItems][kU];
    auto read_o = [&](int u0) {
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int idx = min(threadIdx.x + it * NT, HPW * D - 1);
        const bool item = threadIdx.x + it * NT < HPW * D;
        const int j = idx / D, d = idx % D;
        const int64_t base = (static_cast<int64_t>(b) * H + h0 + j) * p.num_splits + c0;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int uu = u0 + u;
          oa[it][u] = &p.part_o[(base + min(uu, cnt_c - 1)) * D + d];
          ow[it][u] = item && uu < cnt_c && c0 + uu != split ? peek_partial(oa[it][u]) : 1u;
        }
      }
    };
    read_o(0);
    await_partials(ma, mw, oa[0], ow[0], budget);  // (the (m, l) pair and the first o words together)
    if (own_ml) {
      clear_partial(ma[0]);
      clear_partial(ma[1]);
    }
    const bool mine = um < cnt_c && c0 + um == split;
    sm_sm[jm][um] = um < cnt_c ? (mine ? sm_ml[jm][0] : __uint_as_float(mw[0])) : -INFINITY;
    sm_sl[jm][um] = um < cnt_c ? (mine ? sm_ml[jm][1] : __uint_as_float(mw[1])) : 0.0f;
    __syncthreads();
    float newm[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int j = min(threadIdx.x + it * NT, HPW * D - 1) / D;
      float cm = -INFINITY;
      for (int u = 0; u < cnt_c; ++u) cm = fmaxf(cm, sm_sm[j][u]);
      newm[it] = fmaxf(run_m[it], cm);
      if (newm[it] != -INFINITY) {
        const float f_old = run_m[it] == -INFINITY ? 0.0f : exp2f(run_m[it] - newm[it]);
        num[it] *= f_old;
        den[it] *= f_old;
        run_m[it] = newm[it];
      }
    }
    for (int u0 = 0; u0 < cnt_c; u0 += kU) {
      if (u0 > 0) read_o(u0);
#pragma unroll
      for (int it = 0; it < kItems; ++it) await_partials(oa[it], ow[it], budget);
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int idx = threadIdx.x + it * NT;
        if (idx >= HPW * D) break;
        const int j = idx / D, d = idx % D;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int uu = u0 + u;
          if (uu >= cnt_c) break;
          const bool own = c0 + uu == split;
          if (!own) clear_partial(oa[it][u]);
          if (newm[it] == -INFINITY) continue;
          const float ms = sm_sm[j][uu];
          const float f = ms == -INFINITY ? 0.0f : exp2f(ms - newm[it]);
          num[it] = fmaf(own ? sm_o[j][d] : __uint_as_float(ow[it][u]), f, num[it]);
          den[it] = fmaf(sm_sl[j][uu], f, den[it]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int idx = threadIdx.x + it * NT;
    if (idx >= HPW * D) break;
    const int j = idx / D, d = idx % D;
    const float v = den[it] > 0.0f ? num[it] / den[it] : 0.0f;
    p.out[(static_cast<int64_t>(b) * H + h0 + j) * D + d] = f32_to_bf16_rne(v);
  }
}

// Per-wave (m, l, o) in LDS -> the workgroup's (m, l, o): o and l of each
// wave are relative to 2^m of that wave, so they combine with 2^(m_w - M).
template <int D, int HPW, int NW, int NT>
__device__ __forceinline__ void combine_waves(const float (*sm_fo)[HPW][D], const float (*sm_fml)[HPW][2],
                                              float (*sm_o)[D], float (*sm_ml)[2]) {
  for (int idx = threadIdx.x; idx < HPW * D; idx += NT) {
    const int j = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_fml[w][j][0]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_fml[w][j][0];
      if (mw == -INFINITY) continue;
      const float f = exp2f(mw - M);
      acc = fmaf(sm_fo[w][j][d], f, acc);
      lsum = fmaf(sm_fml[w][j][1], f, lsum);
    }
    sm_o[j][d] = acc;
    if (d == 0) {
      sm_ml[j][0] = M;
      sm_ml[j][1] = lsum;
    }
  }
}

// ---------------------------------------------------------------------------
// Recent window (abaddon 0.2.0-rc.1 kv_cache_quant_cuda.rs,
// `OptimizedQuantizedKvCache::get_kv`: the unquantized recent rows follow the
// dequantized old ones).  Positions [L - W, L) are bf16 rows in ring slots
// position % rcap.  The workgroup of the last INT8 split attends to them too:
// after its INT8 blocks, each wave takes 16-token chunks of the ring (loads
// of a chunk in flight together; two dims per lane; fp32 arithmetic with an
// exact running maximum) and merges the result into its own (m, l, o) in
// LDS, which the wave combine then sums as usual.  The fused step's new row
// (position L - 1) comes from the input, rounded to bf16, and is stored in
// its ring slot by the wave that attends to it.
// ---------------------------------------------------------------------------
template <int D, int HPW, bool APPEND>
__device__ void ring_into_wave(const DecodeParams& p, int b, int kvh, int h0, int wave, int lane, int L, int L8,
                               float (*fo)[D], float (*fml)[2], float* scratch) {
  constexpr int kChunk = 16;            // tokens per wave pass
  constexpr int kQ = kWave / kChunk;    // lanes per token for the scores
  constexpr int kDQ = D / kQ;           // dims per lane for the scores
  const int H = p.num_heads;
  // this wave's LDS: fp32 queries [HPW][D], then the pass's weights [16] x 4
  float* sq = scratch;
  float4* sw = reinterpret_cast<float4*>(scratch + HPW * D);
  const bool on = lane < D / 2;         // value lanes: dims (2 lane, 2 lane + 1)
  const int d0 = 2 * (on ? lane : 0);
  const int tt = lane / kQ, qd = lane % kQ;
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    if (on) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p.q + (static_cast<int64_t>(b) * H + h0 + j) * D + d0);
      sq[j * D + d0] = __uint_as_float(w << 16);
      sq[j * D + d0 + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
  float m[HPW], l[HPW], o0[HPW], o1[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    o0[j] = 0.0f;
    o1[j] = 0.0f;
  }
  const int64_t ring0 = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.rcap;
  const int64_t new0 = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * D;
  for (int c0 = L8 + wave * kChunk; c0 < L; c0 += kStreamWaves * kChunk) {
    // scores: token c0 + tt, dims [qd kDQ, (qd + 1) kDQ)
    const int t = c0 + tt;
    const int tc = min(t, L - 1);
    uint32_t kq[kDQ / 2];
    {
      const uint16_t* kr = p.rk + (ring0 + tc % p.rcap) * D + qd * kDQ;
#pragma unroll
      for (int u = 0; u < kDQ / 2; u += 4)
        *reinterpret_cast<uint4*>(&kq[u]) = *reinterpret_cast<const uint4*>(kr + 2 * u);
    }
    // values: this lane's dim pair of the pass's 16 tokens
    uint32_t vw[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      vw[i] = *reinterpret_cast<const uint32_t*>(p.rv + (ring0 + min(c0 + i, L - 1) % p.rcap) * D + d0);
    if constexpr (APPEND) {
      // the new row (position L - 1): from the input, rounded to bf16, and
      // stored in its ring slot
      const int inew = L - 1 - c0;
      if (inew >= 0 && inew < kChunk) {
        uint32_t nk, nv;
        if (p.new_bf16) {
          nk = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.new_k) + new0 + d0);
          nv = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.new_v) + new0 + d0);
        } else {
          const float2 fk = *reinterpret_cast<const float2*>(static_cast<const float*>(p.new_k) + new0 + d0);
          const float2 fv = *reinterpret_cast<const float2*>(static_cast<const float*>(p.new_v) + new0 + d0);
          nk = f32_to_bf16_rne(fk.x) | (static_cast<uint32_t>(f32_to_bf16_rne(fk.y)) << 16);
          nv = f32_to_bf16_rne(fv.x) | (static_cast<uint32_t>(f32_to_bf16_rne(fv.y)) << 16);
        }
        if (on) {
          const int64_t off = (ring0 + (L - 1) % p.rcap) * D + d0;
          *reinterpret_cast<uint32_t*>(p.rk + off) = nk;
          *reinterpret_cast<uint32_t*>(p.rv + off) = nv;
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) vw[u] = u == inew ? nv : vw[u];
        if (tt == inew) {  // this token's score lanes take their K dims from the input
#pragma unroll
          for (int u = 0; u < kDQ / 2; ++u) {
            const int d = qd * kDQ + 2 * u;
            if (p.new_bf16) {
              kq[u] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.new_k) + new0 + d);
            } else {
              const float2 fk = *reinterpret_cast<const float2*>(static_cast<const float*>(p.new_k) + new0 + d);
              kq[u] = f32_to_bf16_rne(fk.x) | (static_cast<uint32_t>(f32_to_bf16_rne(fk.y)) << 16);
            }
          }
        }
      }
    }
    float sc[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < kDQ / 2; ++u) {
        const float2 qq = *reinterpret_cast<const float2*>(sq + j * D + qd * kDQ + 2 * u);
        acc = fmaf(qq.x, __uint_as_float(kq[u] << 16), acc);
        acc = fmaf(qq.y, __uint_as_float(kq[u] & 0xffff0000u), acc);
      }
      acc += __shfl_xor(acc, 1, kWave);  // sum over the token's 4 lanes
      acc += __shfl_xor(acc, 2, kWave);
      sc[j] = t < L ? acc * p.scale_log2 : -INFINITY;
    }
    // softmax over the pass, one reduction per head
    float4 wt = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const float cm = uniform(wave_max(sc[j]));
      const float mn = fmaxf(m[j], cm);
      const float f = m[j] == -INFINITY ? 0.0f : exp2f(m[j] - mn);
      const float w = t < L ? exp2f(sc[j] - mn) : 0.0f;
      l[j] = fmaf(l[j], f, uniform(wave_sum(qd == 0 ? w : 0.0f)));
      o0[j] *= f;
      o1[j] *= f;
      m[j] = mn;
      (&wt.x)[j] = w;
    }
    if (qd == 0) sw[tt] = wt;
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (c0 + i >= L) continue;  // uniform
      const float4 wi = sw[i];
      const float vx = __uint_as_float(vw[i] << 16), vy = __uint_as_float(vw[i] & 0xffff0000u);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        o0[j] = fmaf((&wi.x)[j], vx, o0[j]);
        o1[j] = fmaf((&wi.x)[j], vy, o1[j]);
      }
    }
    wave_lds_sync();  // the next pass rewrites the weights
  }
  // merge into this wave's (m, l, o): both are relative to their own 2^m
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const float m1 = fml[j][0], l1 = fml[j][1];
    const float M = fmaxf(m1, m[j]);
    const float f1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
    const float f2 = m[j] == -INFINITY ? 0.0f : exp2f(m[j] - M);
    if (on) {
      fo[j][d0] = fmaf(fo[j][d0], f1, o0[j] * f2);
      fo[j][d0 + 1] = fmaf(fo[j][d0 + 1], f1, o1[j] * f2);
    }
    wave_lds_sync();  // every lane has read fml[j] before lane 0 rewrites it
    if (lane == 0) {
      fml[j][0] = M;
      fml[j][1] = fmaf(l1, f1, l[j] * f2);
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming kernel (head_dim 32, 64, 128, 256).
// ---------------------------------------------------------------------------
// SM: scale mode (kSmToken fp32 per token, kSmGroup32, kSmTokenBf16 bf16 per
// token), a template argument so each mode pays only for its own decoding
// WIN: a sliding window (p.window > 0), a template argument so that the
// plain kernel's code holds no path where the first block's loads wait for
// the length (the compiler's wait counts after such a join are conservative)
template <int D, int HPW, int SM, bool PAGED, bool APPEND, bool WIN>
__global__ __launch_bounds__(kStreamThreads, 2) void decode_stream_kernel(DecodeParams p) {
  // BLK: tokens per wave block, 8-16 KB of K and V: 64 at head dims 32 and
  // 64, 32 at 128 and 256.  At head dim 128 the 32-token block (8 KB) beats
  // the 64-token one: the block the wave computes after its last loads land
  // is shorter, and the registers fall from about 220 to 160.  (16 tokens
  // was slower again: the per-block softmax and exchange steps dominate.)
  constexpr int BLK = D >= 128 ? 32 : kBlock;
  // K side: a token row is read by LK lanes, 16 bytes each (TK rows per pass).
  // V side: a token row is read by LV lanes, 8 bytes each (TV rows per pass),
  // so a lane accumulates 8 output dims per head.
  constexpr int LK = D / 16, TK = kWave / LK, NPK = BLK / TK;
  constexpr int LV = D / 8, TV = kWave / LV, NPV = BLK / TV;
  constexpr int NPAIR = NPV / 2;             // token pairs per lane per block
  constexpr bool G32 = SM == kSmGroup32;
  constexpr bool SBF = SM == kSmTokenBf16;
  // FP8 codes: values, not offsets from 128, and no scales
  constexpr bool FP8 = SM == kSmFp8E4M3 || SM == kSmFp8E5M2;
  constexpr bool E5 = SM == kSmFp8E5M2;
  constexpr int NG = G32 ? D / 32 : 1;       // scales per row
  constexpr int kSwz = 16 / LK;              // partial-score swizzle
  // MQK: the scores on the matrix cores (v_mfma_f32_16x16x32_f16; head dims
  // 64, 128 and 256): KST k-steps of 32 dims, NU 16-byte K pieces per lane
  // and 16-token group.  A lane's k-slots 8(l/16) + e of k-step s are dims
  // 64(s/2) + 16(l/16) + 8(s%2) + e, so that the four lane groups of one
  // load read a row's 64 contiguous bytes; with group-32 scales they are
  // dims 32s + 8(l/16) + e, so that k-step s is group s.
  constexpr bool MQK = D == 128 || D == 64 || D == 256;
  constexpr int KST = D / 32, NU = D / 64, NGRP = BLK / 16;  // NGRP: 16-token groups per block
  static_assert(NPV % 2 == 0 && LV <= 32, "block shape");
  static_assert(HPW >= 1 && HPW <= 4, "at most four heads per workgroup");

  // partial scores, [k-lane][token ^ (k-lane * 16/LK)] x 4 heads: the writes of
  // one pass and the reads of one k-lane both touch distinct banks
  __shared__ float4 sm_part[kStreamWaves][BLK * LK];
  __shared__ uint4 sm_w[kStreamWaves][NPAIR * TV * NG];    // f16 weight pairs [pair][slot][group] x 4 heads
  __shared__ float sm_fo[kStreamWaves][HPW][D];            // per-wave outputs
  __shared__ float sm_fml[kStreamWaves][HPW][2];           // per-wave (m, l)
  __shared__ float sm_o[HPW][D];                     // workgroup outputs
  __shared__ float sm_ml[HPW][2];
  __shared__ uint4 sm_nk[D / 16];                    // fused append: new K codes
  __shared__ uint2 sm_nv[D / 8];                     // fused append: new V codes
  __shared__ float sm_ns[2][NG];                     // fused append: new K / V scales
  __shared__ int sm_prog[kStreamWaves];              // blocks each wave has started
  __shared__ int sm_last;                            // this split merges the sequence's splits

  // Consecutive workgroup ids go to consecutive XCDs, so the head group varies
  // fastest: each XCD then receives one head group of every (sequence, split),
  // the same token count whatever the mix of lengths.  Head group hg is KV
  // head hg % KVH, query heads (hg / KVH) * HPW onwards of its GQA group:
  // when KVH is a multiple of 8 the workgroups that share a KV head's rows
  // then share an XCD and its L2.
  const int hg = blockIdx.x;
  const int split = blockIdx.y;
  int known_len;  // (the ranking's scratch lies in wave 0's score staging)
  const int b = sequence_of<kStreamThreads>(p, reinterpret_cast<int*>(&sm_part[0][0]), known_len);
  const int H = p.num_heads;
  const int kvh = hg % p.geom.kvh;
  const int h0 = kvh * (H / p.geom.kvh) + (hg / p.geom.kvh) * HPW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int ksub = lane % LK, kslot = lane / LK;     // K lanes: 16 dims of token slot
  const int mtok = lane % 16, mgrp = lane / 16;      // MQK lanes: token of a 16-token group, a quarter of the k-slots
  const int vsub = lane % LV, vslot = lane / LV;     // V lanes: 8 dims of token slot

  // With a sliding window the token range starts at the window's first key,
  // rounded down to a block (blocks stay page-aligned; keys below the window
  // are masked), so it is known only with the length.
  int t_begin = split * p.split_len;
  int t_min = 0;  // first visible key
  // Until seq_lens[b] arrives, t_end is only bounded by the launch: the first
  // block's loads go out against that bound (rows past the real end are valid
  // memory and are masked later), overlapping the length and query loads.
  // A length already read by the ranking bounds them (an empty split loads
  // nothing).
  int t_end = min(known_len >= 0 ? max(known_len - p.rwin, 0) : p.len_cap, t_begin + p.split_len);
  int pn = -1;            // fused append: position of the new row (set once the length is known)
  bool owns_new = false;  // fused append: this workgroup's split holds it

  uint32_t qp[HPW][8];
  // MQK: the queries as the score product's A operand, per k-step; at head
  // dim 256 (where registers are short) they wait in LDS, one copy per
  // workgroup, read once per k-step and block
  constexpr bool kQaLds = D == 256;
  __shared__ half8_t sm_qa[kQaLds ? KST : 1][kQaLds ? kWave : 1];
  half8_t qa[MQK && !kQaLds ? KST : 1];
  auto q_operand = [&](int st) -> half8_t {
    if constexpr (kQaLds) return sm_qa[st][lane];
    else return qa[MQK ? st : 0];
  };
  float fold_row[HPW];  // per-token: 128 * 2^-24 * (sum of the scaled queries), wave-uniform
  float cst[HPW];       // scale_log2 * 2^24 * 2^-kq (wave-uniform)

  // ---- state -------------------------------------------------------------------
  float o[HPW][8];
  float m[HPW], l[HPW], ws[HPW][1];   // weight sums (for the -128 fold)
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    ws[j][0] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.0f;
  }

  uint4 kb[NPK];
  uint2 vb[NPV];
  constexpr int kPidAhead = 4;  // paged: blocks of page ids held ahead (covers a 2048-token split)
  int32_t pq[kPidAhead][BLK / kPageSize] = {};
  float s_k[NG];        // K scales of this lane's softmax token (per token or per group)
  float s_v[NG];        // V scales of this lane's softmax token
  // per-token: the scale words as loaded (fp32, or the aligned word holding a
  // bf16 scale), decoded only where the softmax uses them so that the
  // prefetch is not waited for early; which half holds a bf16 scale follows
  // from the parity of the token's row, recomputed there
  uint32_t s_kw = 0u, s_vw = 0u;
  const int vgroup = G32 ? vsub / 4 : 0;
  const int64_t seq_row0 = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.geom.max_len;
  const uint32_t koff = static_cast<uint32_t>(kslot * D + ksub * 16);   // lane's byte offset in a K pass
  const uint32_t voff = static_cast<uint32_t>(vslot * D + vsub * 8);    // lane's byte offset in a V pass

  // ---- loads --------------------------------------------------------------------
  // A block whose BLK tokens all lie before t_end takes the fast path: the rows of
  // one pass are consecutive (contiguous layout) or lie in one 16-token page
  // (paged layout), so a load is a uniform base plus a per-lane constant.
  // Page ids come from a queue of scalar registers filled kPidAhead blocks
  // ahead with s_load (counted by lgkmcnt, so waiting for them never drains
  // the vector loads in flight).  The last, partial block clamps every
  // row into [t_begin, t_end) instead (paged layouts need no clamp: rows past
  // the end still lie in the block's pages); the extra tokens are discarded
  // through their -inf score and zero weight.  No load sits under a per-lane
  // branch.
  constexpr bool kPassInPage = TK <= kPageSize && TV <= kPageSize;
  constexpr int kPages = BLK / kPageSize;          // pages per block
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const const_i32* bt_s = (const const_i32*)(p.geom.block_table);  // scalar loads
  // page ids of block bi (uniform; ids past the table read as 0)
  auto fetch_pids = [&](int bi, int32_t (&pid)[kPages]) {
    const int blk0 = (t_begin + bi * BLK) >> 4;
#pragma unroll
    for (int pg = 0; pg < kPages; ++pg)
      pid[pg] = blk0 + pg < p.geom.max_blocks ? bt_s[static_cast<int64_t>(b) * p.geom.max_blocks + blk0 + pg] : 0;
  };
  auto page_row0 = [&](int32_t phys) -> int64_t {     // row of a page's slot 0 (uniform)
    phys = min(max(phys, 0), p.geom.num_pages - 1);
    return (static_cast<int64_t>(phys) * p.geom.kvh + kvh) * kPageSize;
  };
  // clamped per-lane row of token t of the block starting at s0 (whose page ids
  // are pid): the clamp keeps t inside the block, so no table read is needed
  auto block_row = [&](int s0, int t, const int32_t (&pid)[kPages]) -> int64_t {
    t = max(min(t, t_end - 1), 0);  // (row 0 stands in when the range is empty)
    if constexpr (PAGED) {
      // the ids are uniform: reading them through readfirstlane makes the
      // per-lane choice a select of values, which the optimiser would otherwise
      // turn into a load at a per-lane index (forcing the queue out of registers)
      const int pg = (t - s0) >> 4;
      int32_t my = __builtin_amdgcn_readfirstlane(pid[0]);
#pragma unroll
      for (int k = 1; k < kPages; ++k) my = pg == k ? __builtin_amdgcn_readfirstlane(pid[k]) : my;
      return page_row0(my) + (t & (kPageSize - 1));
    } else {
      return seq_row0 + t;
    }
  };
  auto row_of = [&](int t) -> int64_t {                  // clamped per-lane row (table read)
    t = max(min(t, t_end - 1), 0);  // (row 0 stands in when the range is empty)
    if constexpr (PAGED) {
      int phys = p.geom.block_table[static_cast<int64_t>(b) * p.geom.max_blocks + (t >> 4)];
      phys = min(max(phys, 0), p.geom.num_pages - 1);
      return (static_cast<int64_t>(phys) * p.geom.kvh + kvh) * kPageSize + (t & (kPageSize - 1));
    } else {
      return seq_row0 + t;
    }
  };
  // K and V code loads: non-temporal, except in the paged layout (where, on
  // the paged workload, they made the step slower)
  auto ld_kv16 = [&](const uint8_t* ptr) -> uint4 {
    if constexpr (PAGED) return *reinterpret_cast<const uint4*>(ptr);
    else return load_stream16(ptr);
  };
  auto ld_kv8 = [&](const uint8_t* ptr) -> uint2 {
    if constexpr (PAGED) return *reinterpret_cast<const uint2*>(ptr);
    else return load_stream8(ptr);
  };
  auto load_scales = [&](int64_t srow) {
    if constexpr (FP8) {
      (void)srow;
    } else if constexpr (NG == 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(p.k_scales + srow * NG);
      const float4 v4 = *reinterpret_cast<const float4*>(p.v_scales + srow * NG);
      s_k[0] = k4.x; s_k[1] = k4.y; s_k[2] = k4.z; s_k[3] = k4.w;
      s_v[0] = v4.x; s_v[1] = v4.y; s_v[2] = v4.z; s_v[3] = v4.w;
    } else if constexpr (G32) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        s_k[g] = p.k_scales[srow * NG + g];
        s_v[g] = p.v_scales[srow * NG + g];
      }
    } else {
      s_kw = scale_word(p.k_scales, srow, SBF);
      s_vw = scale_word(p.v_scales, srow, SBF);
    }
  };
  // scales of the softmax token (token `lane`) of block bi
  // (scales of rows past the end could be any bits, so their rows are clamped)
  auto load_block_scales = [&](int bi, const int32_t (&pid)[kPages]) {
    const int s0 = t_begin + bi * BLK;
    load_scales(block_row(s0, s0 + lane, pid));
  };
  auto load_k = [&](int bi, const int32_t (&pid)[kPages]) {
    const int s0 = t_begin + bi * BLK;
    if constexpr (MQK) {
      // lane l: token 16g + l % 16 of each 16-token group g (one page), 16
      // bytes at 64u + 16(l / 16) for each u, or (group-32) 8 bytes of each
      // group
      auto piece = [&](int64_t r, int g) {
        const uint8_t* row = p.k_codes + r * D;
        if constexpr (G32) {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            // (plain loads: two instructions read each 64-byte segment, and a
            // non-temporal first read lets the line go before the second)
            const uint2 a = *reinterpret_cast<const uint2*>(row + 64 * u + 8 * mgrp);
            const uint2 c = *reinterpret_cast<const uint2*>(row + 64 * u + 32 + 8 * mgrp);
            kb[g * NU + u] = make_uint4(a.x, a.y, c.x, c.y);
          }
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u) kb[g * NU + u] = ld_kv16(row + 64 * u + 16 * mgrp);
        }
      };
      if (PAGED || s0 + BLK <= t_end) {
#pragma unroll
        for (int g = 0; g < NGRP; ++g) piece(PAGED ? page_row0(pid[g]) + mtok : seq_row0 + s0 + 16 * g + mtok, g);
      } else {
#pragma unroll
        for (int g = 0; g < NGRP; ++g) piece(row_of(s0 + 16 * g + mtok), g);
      }
      return;
    }
    if (PAGED ? kPassInPage : s0 + BLK <= t_end) {
      if constexpr (PAGED) {
        int64_t r0[kPages];
#pragma unroll
        for (int pg = 0; pg < kPages; ++pg) r0[pg] = page_row0(pid[pg]);
#pragma unroll
        for (int i = 0; i < NPK; ++i) {
          const int tok = i * TK;                          // first token of the pass
          const uint8_t* base = p.k_codes + (r0[tok >> 4] + (tok & 15)) * D;
          kb[i] = ld_kv16(base + koff);
        }
      } else {
        const int64_t r = seq_row0 + s0;
        const uint8_t* base = p.k_codes + r * D;
#pragma unroll
        for (int i = 0; i < NPK; ++i) {
          kb[i] = ld_kv16(base + i * TK * D + koff);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPK; ++i) {
        const int64_t row = row_of(s0 + i * TK + kslot);
        kb[i] = ld_kv16(p.k_codes + row * D + ksub * 16);
      }
    }
  };
  auto load_v = [&](int bi, const int32_t (&pid)[kPages]) {
    const int s0 = t_begin + bi * BLK;
    if (PAGED ? kPassInPage : s0 + BLK <= t_end) {
      if constexpr (PAGED) {
        int64_t r0[kPages];
#pragma unroll
        for (int pg = 0; pg < kPages; ++pg) r0[pg] = page_row0(pid[pg]);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int tok = i * TV;
          const uint8_t* base = p.v_codes + (r0[tok >> 4] + (tok & 15)) * D;
          vb[i] = ld_kv8(base + voff);
        }
      } else {
        const uint8_t* base = p.v_codes + (seq_row0 + s0) * D;
#pragma unroll
        for (int i = 0; i < NPV; ++i) vb[i] = ld_kv8(base + i * TV * D + voff);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int64_t row = row_of(s0 + i * TV + vslot);
        vb[i] = ld_kv8(p.v_codes + row * D + vsub * 8);
      }
    }
  };

  // ---- one block of BLK tokens; PREFETCH issues the next block's loads early ------
  // Waves w and w + 4 share a SIMD, whose issue arbitration favours the older
  // one: left alone it finishes its blocks well ahead of the younger, which
  // then streams by itself.  With long splits over ragged lengths (several
  // rounds of workgroups, where the last ones stream alone and a workgroup's
  // own rate decides) a wave that has started fewer blocks than its partner
  // takes the higher priority, so the two keep pace (measured on the paged
  // workload: 2-4% faster).  With one round the chip's bandwidth is the limit
  // and the check only costs time; the contiguous kernel leaves it out, since
  // even untaken it slows the loop's code by 3%.  (Scheduling only: which
  // wave computes which block is unchanged.)
  int started = 0;
  volatile int* prog = sm_prog;
  if (PAGED && p.balance && lane == 0) prog[wave] = 0;
  auto run_block = [&](int blk, auto prefetch) {
    constexpr bool PREFETCH = decltype(prefetch)::value;
    if (PAGED && p.balance) {
      ++started;
      if (lane == 0) prog[wave] = started;
      if (started < __builtin_amdgcn_readfirstlane(prog[wave ^ (kStreamWaves / 2)])) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (APPEND) {
      // the block holding the freshly appended token uses the codes just
      // computed (its loads may have been issued before they were stored)
      const int s0 = t_begin + blk * BLK;
      if (owns_new && pn >= s0 && pn < s0 + BLK) {
        const int rel = pn - s0;
        if constexpr (MQK) {
          const uint2* nk2 = reinterpret_cast<const uint2*>(sm_nk);
#pragma unroll
          for (int g = 0; g < NGRP; ++g)
            if (16 * g + mtok == rel) {
#pragma unroll
              for (int u = 0; u < NU; ++u) {
                if constexpr (G32) {
                  const uint2 a = nk2[8 * u + mgrp], c = nk2[8 * u + 4 + mgrp];
                  kb[g * NU + u] = make_uint4(a.x, a.y, c.x, c.y);
                } else {
                  kb[g * NU + u] = sm_nk[4 * u + mgrp];
                }
              }
            }
        } else {
#pragma unroll
          for (int i = 0; i < NPK; ++i) {
            if (i * TK + kslot == rel) {
              kb[i] = sm_nk[ksub];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NPV; ++i)
          if (i * TV + vslot == rel) vb[i] = sm_nv[vsub];
        if (lane == rel) {
          if constexpr (G32) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              s_k[g] = sm_ns[0][g];
              s_v[g] = sm_ns[1][g];
            }
          } else if constexpr (!FP8) {
            // a stored bf16 scale has a zero low half: copied into both
            // halves it decodes the same whichever half is selected
            const uint32_t nk = __float_as_uint(sm_ns[0][0]), nv = __float_as_uint(sm_ns[1][0]);
            s_kw = SBF ? nk | (nk >> 16) : nk;
            s_vw = SBF ? nv | (nv >> 16) : nv;
          }
        }
      }
    }
    float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MQK) {
      // S = Q K^T per 16-token group: A = the queries (rows: heads, HPW of
      // 16 used), B = K^T (lane l: token l % 16, k-slots 8(l/16) + e, the
      // same dims of k-step s as for the queries).  The
      // result's row 4(l/16) + i, column l % 16 puts heads 0..3 of the
      // group's tokens in lanes 0..15.
      auto k_operand = [&](int g, int st) {
        const uint4 w = kb[g * NU + st / 2];
        const uint32_t w0 = (st & 1) ? w.z : w.x, w1 = (st & 1) ? w.w : w.y;
        uint32_t c4[4];
        if constexpr (G32) {  // exact f16 c - 128: the group scale multiplies later
          c4[0] = exact_pair(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u));
          c4[1] = exact_pair(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u));
          c4[2] = exact_pair(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u));
          c4[3] = exact_pair(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u));
        } else if constexpr (FP8) {
          c4[0] = fp8_pair_k<E5, false>(w0);
          c4[1] = fp8_pair_k<E5, true>(w0);
          c4[2] = fp8_pair_k<E5, false>(w1);
          c4[3] = fp8_pair_k<E5, true>(w1);
        } else {
          c4[0] = __builtin_amdgcn_perm(0u, w0, 0x0C010C00u);
          c4[1] = __builtin_amdgcn_perm(0u, w0, 0x0C030C02u);
          c4[2] = __builtin_amdgcn_perm(0u, w1, 0x0C010C00u);
          c4[3] = __builtin_amdgcn_perm(0u, w1, 0x0C030C02u);
        }
        return __builtin_bit_cast(half8_t, c4);
      };
      // group g's scores to lanes 16g .. 16g + 15: rows of 16 lanes swap
      // pairwise (row 1 of the first operand with row 0 of the second),
      // then halves (two groups: the first swap alone)
      auto gather = [&](const float4_t (&sg)[NGRP], int j) {
        const uint32_t y01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sg[0][j]), __float_as_uint(sg[1][j]),
                                                               false, false)[0];
        if constexpr (NGRP == 2) {
          return __uint_as_float(y01);
        } else {
          const uint32_t y23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sg[2][j]), __float_as_uint(sg[3][j]),
                                                                 false, false)[0];
          return __uint_as_float(__builtin_amdgcn_permlane32_swap(y01, y23, false, false)[0]);
        }
      };
      if constexpr (G32) {
        // one k-step per group: its partial scores, gathered, times the
        // token's group scale
#pragma unroll
        for (int st = 0; st < KST; ++st) {
          float4_t sg[NGRP];
          const half8_t a = q_operand(st);
#pragma unroll
          for (int g = 0; g < NGRP; ++g)
            sg[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, k_operand(g, st), float4_t{0.0f, 0.0f, 0.0f, 0.0f},
                                                            0, 0, 0);
#pragma unroll
          for (int j = 0; j < HPW; ++j) S[j] = fmaf(gather(sg, j), s_k[st], S[j]);
        }
      }
      // (the groups' products interleave: NGRP independent accumulators)
      float4_t sg[NGRP];
#pragma unroll
      for (int g = 0; g < NGRP; ++g) sg[g] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < (G32 ? 0 : KST); ++st) {
        const half8_t a = q_operand(st);
#pragma unroll
        for (int g = 0; g < NGRP; ++g) sg[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, k_operand(g, st), sg[g], 0, 0, 0);
      }
      if constexpr (!G32) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) S[j] = gather(sg, j);
      }
    }
    // QK: partial dots of this lane's 16 dims, all heads
#pragma unroll
    for (int i = 0; i < (MQK ? 0 : NPK); ++i) {
      const uint32_t kw[4] = {kb[i].x, kb[i].y, kb[i].z, kb[i].w};
      float P[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        uint32_t c01, c23;
        if constexpr (G32) {
          // exact f16 c - 128: the group scale multiplies the partial later
          c01 = exact_pair(__builtin_amdgcn_perm(0x64646464u, kw[w4], 0x04010400u));
          c23 = exact_pair(__builtin_amdgcn_perm(0x64646464u, kw[w4], 0x04030402u));
        } else if constexpr (FP8) {
          c01 = fp8_pair_k<E5, false>(kw[w4]);
          c23 = fp8_pair_k<E5, true>(kw[w4]);
        } else {
          c01 = __builtin_amdgcn_perm(0u, kw[w4], 0x0C010C00u);
          c23 = __builtin_amdgcn_perm(0u, kw[w4], 0x0C030C02u);
        }
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          P[j] = dot2(qp[j][2 * w4], c01, P[j]);
          P[j] = dot2(qp[j][2 * w4 + 1], c23, P[j]);
        }
      }
      sm_part[wave][ksub * BLK + ((i * TK + kslot) ^ (ksub * kSwz))] = make_float4(P[0], P[1], P[2], P[3]);
    }
    if constexpr (PREFETCH) load_k(blk + kStreamWaves, pq[1]);
    if constexpr (!MQK) wave_lds_sync();

    // softmax: this lane owns token `lane` of the block
    const int t = t_begin + blk * BLK + lane;
    const bool valid = t < t_end && t >= t_min && lane < BLK;
    float4 acc4 = MQK ? make_float4(S[0], S[1], S[2], S[3]) : sm_part[wave][lane ^ 0];
    if constexpr (!G32 && !FP8) {
      // the row of the (clamped) token: page rows start even, so in the paged
      // layout its parity is the token's
      const int tc = min(t, t_end - 1);
      const uint32_t sel = scale_sel(PAGED ? static_cast<int64_t>(tc) : seq_row0 + tc, SBF);
      s_k[0] = scale_value(s_kw, sel);
      s_v[0] = scale_value(s_vw, sel);
    }
    if constexpr (G32 && !MQK) acc4 = make_float4(acc4.x * s_k[0], acc4.y * s_k[0], acc4.z * s_k[0], acc4.w * s_k[0]);
#pragma unroll
    for (int r = 1; r < (MQK ? 1 : LK); ++r) {
      const float4 v = sm_part[wave][r * BLK + (lane ^ (r * kSwz))];
      if constexpr (G32) {
        const float sg = s_k[r >> 1];  // k-lane r holds dims 16r..16r+15: group r / 2
        acc4.x = fmaf(v.x, sg, acc4.x); acc4.y = fmaf(v.y, sg, acc4.y);
        acc4.z = fmaf(v.z, sg, acc4.z); acc4.w = fmaf(v.w, sg, acc4.w);
      } else {
        acc4.x += v.x; acc4.y += v.y; acc4.z += v.z; acc4.w += v.w;
      }
    }
    S[0] = acc4.x; S[1] = acc4.y; S[2] = acc4.z; S[3] = acc4.w;
    // V scale of the token: per-token, or the largest of its groups (group-32)
    float sv_top = FP8 ? 1.0f : s_v[0];
#pragma unroll
    for (int g = 1; g < NG; ++g) sv_top = fmaxf(sv_top, s_v[g]);
    const float lsv_max = FP8 ? 0.0f : __log2f(sv_top);
    float Sh[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      // per-token scales fold the offset once for the whole row, then scale
      const float dotv = G32 || FP8 ? S[j] : (S[j] - fold_row[j]) * s_k[0];
      Sh[j] = valid ? dotv * cst[j] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      // raise the (wave-uniform) reference only when some score exceeds it by
      // more than 2^8; the exact block maximum is needed only then
      if (any_lane(Sh[j] + lsv_max > m[j] + kLazy)) {
        const float bm = uniform(wave_max(Sh[j] + lsv_max));
        const float alpha = fast_exp2(m[j] - bm);
        m[j] = bm;
        l[j] *= alpha;
        ws[j][0] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
      }
    }
    // token lane = V pass * TV + V slot; pair V passes (2k, 2k+1) of one slot:
    // the partner token sits TV lanes higher
    const bool even_pass = ((lane / TV) & 1) == 0;
    const int wslot = ((lane / TV) >> 1) * TV + lane % TV;
    if constexpr (G32) {
      // w_g = 2^(S + log2 sV_g - m + 7) = E * (sV_g / sV_top) with
      // E = 2^(S + log2 sV_top - m + 7) <= 2^15; the normaliser takes
      // 2^(S - m) = E / (128 sV_top).  One exponential per head.  A masked
      // token (E = 0) may come from a row never written, whose scales are
      // 0: its factor is taken as 0, not 1/0, so no 0 * inf enters the sums.
      const float inv = valid ? 1.0f / sv_top : 0.0f;
      float E[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        E[j] = fast_exp2(Sh[j] + lsv_max - m[j] + static_cast<float>(kWeightShift));  // -inf score: 0
        l[j] = fmaf(E[j], inv * 0x1p-7f, l[j]);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float r = s_v[g] * inv;
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          const uint32_t wb = f16_bits(E[j] * r);
          word[j] = wb | (lane_up<TV>(wb) << 16);
        }
        if (even_pass && lane < BLK) sm_w[wave][wslot * NG + g] = make_uint4(word[0], word[1], word[2], word[3]);
      }
    } else {
      uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        l[j] += fast_exp2(Sh[j] - m[j]);  // -inf score: exactly 0
        const uint32_t wb = f16_bits(fast_exp2(Sh[j] + lsv_max - m[j] + static_cast<float>(kWeightShift)));
        if constexpr (!FP8) ws[j][0] += f16_value(wb);
        word[j] = wb | (lane_up<TV>(wb) << 16);
      }
      if (even_pass && lane < BLK) sm_w[wave][wslot] = make_uint4(word[0], word[1], word[2], word[3]);
    }
    // the scales of this block are used up: fetch the next block's
    if constexpr (PREFETCH) load_block_scales(blk + kStreamWaves, pq[1]);
    wave_lds_sync();

    // FP8: a masked token may come from a row never written, whose bytes can
    // be NaN or inf codes; its weight is 0, but 0 * NaN is not, so such rows
    // read as zero codes (blocks wholly inside [t_min, t_end) skip this)
    if constexpr (FP8) {
      const int s0 = t_begin + blk * BLK;
      if (s0 < t_min || s0 + BLK > t_end) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int tv = s0 + i * TV + vslot;
          if (tv < t_min || tv >= t_end) vb[i] = make_uint2(0u, 0u);
        }
      }
    }
    // PV: token pairs, this lane's 8 dims, all heads
#pragma unroll
    for (int k = 0; k < NPAIR; ++k) {
      const uint4 wq = sm_w[wave][(k * TV + vslot) * NG + vgroup];
      const uint32_t wv[4] = {wq.x, wq.y, wq.z, wq.w};
      if constexpr (G32) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) ws[j][0] = dot2(wv[j], 0x3C003C00u, ws[j][0]);  // f16 pair (1, 1)
      }
      const uint32_t a2[2] = {vb[2 * k].x, vb[2 * k].y};
      const uint32_t b2[2] = {vb[2 * k + 1].x, vb[2 * k + 1].y};
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t cp = FP8 ? fp8_pair_v<E5>(a2[w2], b2[w2], e)
                                  : __builtin_amdgcn_perm(b2[w2], a2[w2], 0x0C040C00u + 0x00010001u * e);
#pragma unroll
          for (int j = 0; j < HPW; ++j) o[j][4 * w2 + e] = dot2(wv[j], cp, o[j][4 * w2 + e]);
        }
      }
    }
    if constexpr (PREFETCH) load_v(blk + kStreamWaves, pq[1]);
    if constexpr (PAGED) {  // advance the page-id queue
#pragma unroll
      for (int k = 0; k + 1 < kPidAhead; ++k)
#pragma unroll
        for (int pg = 0; pg < kPages; ++pg) pq[k][pg] = pq[k + 1][pg];
      if (t_begin + (blk + kPidAhead * kStreamWaves) * BLK < t_end) fetch_pids(blk + kPidAhead * kStreamWaves, pq[kPidAhead - 1]);
    }
  };

  // the wave index is uniform, so every block condition below is a scalar branch
  int blk = wave;
  // The length, the fused append's new row and the queries go out before the
  // first block's K/V loads, so they do not queue behind the bulk traffic
  // every workgroup starts with.  The code between these loads and the
  // queries' use holds no loop of memory operations, so the wait for the
  // queries covers the queries alone, not the first block as well (the
  // compiler's wait counts are exact only through straight-line code).
  const int len_raw = p.seq_lens[b];
  // fused append: waves 0 and 1 fetch the new K and V rows of this KV head
  // (with a recent window the row to quantize is the one leaving the ring,
  // fetched once the length is known)
  constexpr int kEpl = row_epl(D);
  uint4 xraw = make_uint4(0u, 0u, 0u, 0u);  // the row's raw bytes, converted where they are quantized
  const bool xbf16 = p.new_bf16 != 0;
  if (APPEND && p.rwin == 0) {
    const size_t esz = xbf16 ? 2 : 4;
    const char* src = static_cast<const char*>(wave == 0 ? p.new_k : p.new_v) +
                      (static_cast<int64_t>(b) * p.geom.kvh + kvh) * D * esz;
    xraw = load_row_raw<kEpl>(src, lane, wave < 2 && lane < D / kEpl, xbf16);
  }
  // (without the matrix cores: LK lanes per query row, 16 dims each)
  uint4 qraw[MQK ? 1 : HPW][2];
  if constexpr (!MQK) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const uint4* qptr = reinterpret_cast<const uint4*>(p.q + (static_cast<int64_t>(b) * H + h0 + j) * D + ksub * 16);
      qraw[j][0] = qptr[0];
      qraw[j][1] = qptr[1];
    }
  }
  // MQK: this lane's operand rows of the score product: head l % 16 (lanes
  // past the HPW heads read head HPW - 1 and later hold zeros), the 8 dims
  // of its k-slots at each k-step s
  uint4 qmr[MQK ? KST : 1];
  if constexpr (MQK) {
    const uint16_t* qrow = p.q + (static_cast<int64_t>(b) * H + h0 + min(mtok, HPW - 1)) * D;
#pragma unroll
    for (int st = 0; st < KST; ++st)
      qmr[st] = *reinterpret_cast<const uint4*>(qrow + (G32 ? 32 * st + 8 * mgrp : 64 * (st / 2) + 16 * mgrp + 8 * (st % 2)));
  }
  auto first_loads = [&]() {
    if constexpr (PAGED) {
#pragma unroll
      for (int k = 0; k < kPidAhead; ++k)
        if (t_begin + (blk + k * kStreamWaves) * BLK < t_end) fetch_pids(blk + k * kStreamWaves, pq[k]);
    }
    // unconditional (rows clamped into the range, row 0 if it is empty), so
    // that every path issues the same loads and the waits after them stay exact
    load_k(blk, pq[0]);
    load_v(blk, pq[0]);
    load_block_scales(blk, pq[0]);
  };
  if constexpr (!WIN) first_loads();  // speculative first block
  const int L = len_raw < 0 ? 0 : (len_raw > p.len_cap ? p.len_cap : len_raw);
  const int L8 = L > p.rwin ? L - p.rwin : 0;  // INT8 tokens (all of them without a recent window)
  int t_base = 0;  // first token of split 0
  if constexpr (WIN) {
    t_min = max(L - p.window, 0);
    t_base = t_min & ~(BLK - 1);
    t_begin = t_base + split * p.split_len;
  }
  const int ns8 = split_count(L8 - t_base, p.split_len);
  // recent window: the workgroup of the last INT8 split (split 0 if there is
  // none) also attends to the ring
  const bool ring_here = p.rwin > 0 && L > 0 && split == (ns8 > 0 ? ns8 - 1 : 0);
  if ((split >= ns8 || t_begin >= L8) && !ring_here) {  // no tokens here (and not counted)
    if (L == 0 && split == 0) {  // empty window: the output is zero
      for (int idx = threadIdx.x; idx < HPW * D; idx += kStreamThreads)
        p.out[(static_cast<int64_t>(b) * H + h0 + idx / D) * D + idx % D] = 0;
    }
    return;
  }
  const int t_end_spec = t_end;
  t_end = split == ns8 - 1 ? L8 : min(L8, t_begin + p.split_len);  // the last split takes the remainder
  const int nblk = t_end > t_begin ? (t_end - t_begin + BLK - 1) / BLK : 0;
  const int ns = ns8 > 0 ? ns8 : 1;
  if constexpr (WIN) {
    // (the first block's loads go out after the queries' prescale, below)
  } else if constexpr (PAGED) {
    // a remainder joined to the last split lies past the speculative bound:
    // fetch the page ids the queue skipped
    if (t_end > t_end_spec) {
#pragma unroll
      for (int k = 0; k < kPidAhead; ++k)
        if (t_begin + (blk + k * kStreamWaves) * BLK < t_end) fetch_pids(blk + k * kStreamWaves, pq[k]);
    }
  }
  // fused append: the workgroup whose split holds position L8 - 1 quantizes
  // the row that enters the INT8 part (abaddon kv_cache_quant_cuda.rs
  // `quantize_tensor` steps), stores it in the cache, and keeps a copy in LDS
  // for its own attention.  Without a recent window that row is the new one;
  // with one it is the ring row at position L - 1 - W, which this step moves
  // out of the window.
  pn = L8 - 1;
  // (per-head block scales: only a row that starts a block has codes to
  // make, its block's; the others were made with their block's first row)
  owns_new = APPEND && pn >= t_begin && pn < t_end && (!p.block_head || pn % kBlockRows == 0);

  // ---- queries: power-of-two prescale into [2^14, 2^15), f16 pairs -----------
#pragma unroll
  for (int j = 0; j < (MQK ? 0 : HPW); ++j) {
    float qf[16];
    bf16x8_to_f32(qraw[j][0], &qf[0]);
    bf16x8_to_f32(qraw[j][1], &qf[8]);
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(qf[e]));
    a = group_max<LK>(a);
    const int kq = a > 0.0f ? 14 - ilogbf(a) : 0;
    float qs = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t b0 = f16_bits(ldexpf(qf[2 * k], kq)), b1 = f16_bits(ldexpf(qf[2 * k + 1], kq));
      qs += f16_value(b0) + f16_value(b1);
      qp[j][k] = b0 | (b1 << 16);
    }
    fold_row[j] = FP8 ? 0.0f : uniform(group_sum<LK>(qs * (128.0f * 0x1p-24f)));
    // INT8 per-token codes enter as c 2^-24; group-32 and FP8 as exact values
    cst[j] = uniform(ldexpf(p.scale_log2, (G32 || FP8 ? 0 : 24) - kq));
  }
  if constexpr (MQK) {
    // The prescale worked out in the score product's lane layout alone: the
    // four lanes l % 16 = j together hold every dim of head j, so one pass
    // over this lane's KST * 8 values gives the head's absmax, its operand
    // and its sum (each wave of the workgroup does it once, instead of once
    // per head in the row layout as well).  The same exponent as from the
    // head's row; the sum of the same f16 values.
    float a = 0.0f;
#pragma unroll
    for (int st = 0; st < KST; ++st) {
      float qf[8];
      bf16x8_to_f32(qmr[st], qf);
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(qf[e]));
    }
    a = slot_max<16>(a);
    const int kqm = a > 0.0f ? 14 - ilogbf(a) : 0;
    float qs = 0.0f;
#pragma unroll
    for (int st = 0; st < KST; ++st) {
      float qf[8];
      bf16x8_to_f32(qmr[st], qf);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b0 = f16_bits(ldexpf(qf[2 * e], kqm)), b1 = f16_bits(ldexpf(qf[2 * e + 1], kqm));
        qs += f16_value(b0) + f16_value(b1);
        w[e] = mtok < HPW ? b0 | (b1 << 16) : 0u;
      }
      if constexpr (kQaLds) {
        if (wave == 0) sm_qa[st][lane] = __builtin_bit_cast(half8_t, w);
      } else {
        qa[st] = __builtin_bit_cast(half8_t, w);
      }
    }
    qs = slot_sum<16>(qs);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {  // head j's figures, from lane j
      const int kq = __builtin_amdgcn_readlane(kqm, j);
      fold_row[j] = FP8 ? 0.0f : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qs), j)) * (128.0f * 0x1p-24f);
      // INT8 per-token codes enter as c 2^-24; group-32 and FP8 as exact values
      cst[j] = uniform(ldexpf(p.scale_log2, (G32 || FP8 ? 0 : 24) - kq));
    }
    if constexpr (kQaLds) __syncthreads();
  }

  // a sliding window's first block, whose range needed the length
  if constexpr (WIN) first_loads();
  // fused append, after the queries' prescale (its stores would otherwise
  // make the wait for the queries cover the first block too)
  if constexpr (APPEND) {
    if (owns_new) {
      // (a sliding window never has a recent window, so WIN kernels leave it out)
      if (SM == kSmToken && !WIN && p.block_head && wave < 2) {
        // Per-head block scales (the leaving row pn starts block pn / 16):
        // one scale over the block's 16 rows, all of them ring rows (with a
        // 15-row window the last is this step's new row, taken from the
        // input as bf16), and each row's codes under it.  Two passes over
        // the rows keep few registers live: the maximum, then the codes.
        // The block lies in one page, so its rows follow row pn.
        const int64_t rbase = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.rcap;
        const char* nsrc = static_cast<const char*>(wave == 0 ? p.new_k : p.new_v) +
                           (static_cast<int64_t>(b) * p.geom.kvh + kvh) * D * (xbf16 ? 2 : 4);
        auto block_row_values = [&](int i, float (&x)[kEpl]) {
          const int pos = pn + i;
          if (pos == L - 1) {
            row_raw_values<kEpl>(load_row_raw<kEpl>(nsrc, lane, lane < D / kEpl, xbf16), xbf16, x);
#pragma unroll
            for (int e = 0; e < kEpl; ++e) x[e] = bf16_to_f32(f32_to_bf16_rne(x[e]));
          } else {
            const uint16_t* src = (wave == 0 ? p.rk : p.rv) + (rbase + pos % p.rcap) * D;
            row_raw_values<kEpl>(load_row_raw<kEpl>(src, lane, lane < D / kEpl, true), true, x);
          }
        };
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < kBlockRows; ++i) {
          float x[kEpl];
          block_row_values(i, x);
#pragma unroll
          for (int e = 0; e < kEpl; ++e) a = fmaxf(a, fabsf(x[e]));
        }
        a = wave_max(a);
        const float sb = fmaxf(a, 1e-8f) / 127.0f;  // IEEE division (correctly rounded)
        const int64_t row0 = row_of(pn);
        uint8_t* codes = wave == 0 ? p.k_codes : p.v_codes;
#pragma unroll 4
        for (int i = 0; i < kBlockRows; ++i) {
          float x[kEpl];
          block_row_values(i, x);
          const uint32_t packed = codes_with_scale<kEpl>(x, sb);
          if (lane < D / kEpl) store_lane_codes<kEpl>(codes + (row0 + i) * D, lane, packed);
          if (lane == 0) store_scale(wave == 0 ? p.k_scales : p.v_scales, row0 + i, sb, false);
          if (i == 0 && lane < D / kEpl)
            store_lane_codes<kEpl>(wave == 0 ? reinterpret_cast<uint8_t*>(sm_nk) : reinterpret_cast<uint8_t*>(sm_nv),
                                   lane, packed);
        }
        if (lane == 0) sm_ns[wave][0] = sb;
      } else if (wave < 2) {
        float xnew[kEpl];
        if (p.rwin > 0) {  // the ring row leaving the window (its own branch: this load is waited for at once)
          const uint16_t* src = (wave == 0 ? p.rk : p.rv) +
                                ((static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.rcap + pn % p.rcap) * D;
          row_raw_values<kEpl>(load_row_raw<kEpl>(src, lane, lane < D / kEpl, true), true, xnew);
        } else {
          row_raw_values<kEpl>(xraw, xbf16, xnew);
        }
        float sc = 0.0f;
        uint32_t packed;
        if constexpr (FP8) packed = fp8_encode_lane<kEpl, E5>(xnew);
        else packed = quantize_lane<kEpl, G32>(xnew, sc);
        const int64_t row = row_of(pn);
        if (lane < D / kEpl) {
          store_lane_codes<kEpl>((wave == 0 ? p.k_codes : p.v_codes) + row * D, lane, packed);
          store_lane_codes<kEpl>(wave == 0 ? reinterpret_cast<uint8_t*>(sm_nk) : reinterpret_cast<uint8_t*>(sm_nv),
                                 lane, packed);
          constexpr int kGroupLanes = 32 / kEpl;
          float* gs = (wave == 0 ? p.k_scales : p.v_scales) + row * NG;
          if (FP8) {
            // no scales
          } else if (G32) {
            if (lane % kGroupLanes == 0) {
              gs[lane / kGroupLanes] = sc;
              sm_ns[wave][lane / kGroupLanes] = sc;
            }
          } else if (lane == 0) {
            sm_ns[wave][0] = store_scale(wave == 0 ? p.k_scales : p.v_scales, row, sc, SBF);
          }
        }
      }
      __syncthreads();
    }
  }

  for (; blk + kStreamWaves < nblk; blk += kStreamWaves) run_block(blk, std::true_type{});
  if (blk < nblk) run_block(blk, std::false_type{});
  if constexpr (PAGED) __builtin_amdgcn_s_setprio(0);

  // the split's merge ticket, drawn by wave 0 as soon as its blocks are done,
  // so that the round trip overlaps the other waves' last blocks.  The
  // increment wraps: the last of the ns tickets returns the counter to zero
  // for the next call.
  uint32_t ticket = 0u;
  if (ns > 1 && threadIdx.x == 0)
    ticket = __builtin_amdgcn_atomic_inc32(reinterpret_cast<uint32_t*>(p.counters) +
                                               static_cast<int64_t>(b) * gridDim.x + hg,
                                           static_cast<uint32_t>(ns - 1), __ATOMIC_RELAXED, "agent");

  // ---- combine the wave: l and weight sums over lanes, o over token slots ------
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    l[j] = wave_sum(l[j]);
    // U = sum_t 2^(S + log2 sV - m) (c - 128) = 2^-7 (2^24 o - 128 sum w);
    // FP8 codes are values: U = sum_t 2^(S - m) v = 2^-7 o.
    // Group-32: each V lane folds the weights it used (its group, its token
    // slot) before the slot sum; per-token: the softmax lanes' sum, folded
    // after it.
    if constexpr (G32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = fmaf(o[j][e], 0x1p17f, -ws[j][0]);
    } else {
      if constexpr (!FP8) ws[j][0] = wave_sum(ws[j][0]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = slot_sum<LV>(o[j][e]);
  }
  if (vslot == 0) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sm_fo[wave][j][vsub * 8 + e] = G32 ? o[j][e] : (FP8 ? o[j][e] * 0x1p-7f : o[j][e] * 0x1p17f - ws[j][0]);
      if (vsub == 0) {
        sm_fml[wave][j][0] = m[j];
        sm_fml[wave][j][1] = l[j];
      }
    }
  }
  if (ring_here) {
    // this wave's INT8 result is in sm_fo / sm_fml; its score staging area is
    // free (only this wave uses it)
    wave_lds_sync();
    ring_into_wave<D, HPW, APPEND>(p, b, kvh, h0, wave, lane, L, L8, sm_fo[wave], sm_fml[wave],
                                   reinterpret_cast<float*>(&sm_part[wave][0]));
  }
  if (threadIdx.x == 0) sm_last = ticket == static_cast<uint32_t>(ns - 1);
  __syncthreads();
  // ---- combine the waves ------------------------------------------------------------
  combine_waves<D, HPW, kStreamWaves, kStreamThreads>(sm_fo, sm_fml, sm_o, sm_ml);
  __syncthreads();
  finish_split<D, HPW, kStreamThreads>(p, b, h0, split, ns, sm_last != 0, sm_o, sm_ml);
}

// Launch of one scale mode's streaming-kernel instantiations (head_dim 32, 64,
// 128, 256; 1, 2 or 4 heads per workgroup; contiguous or paged; plain or fused
// append).  Each mode's instantiations live in a translation unit of their
// own (kvq_decode_<mode>.hip), so the library's kernels compile in parallel.
template <int SM>
void launch_stream_impl(int head_dim, int hpw, bool paged, bool append, const DecodeParams& p, dim3 grid,
                        hipStream_t st) {
  auto go2 = [&](auto dc, auto hc, auto wc) {
    constexpr int D = decltype(dc)::value;
    constexpr int HPW = decltype(hc)::value;
    constexpr bool WIN = decltype(wc)::value;
    if (paged) {
      if (append) hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, true, true, WIN>), grid, dim3(kStreamThreads), 0, st, p);
      else hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, true, false, WIN>), grid, dim3(kStreamThreads), 0, st, p);
    } else {
      if (append) hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, false, true, WIN>), grid, dim3(kStreamThreads), 0, st, p);
      else hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, false, false, WIN>), grid, dim3(kStreamThreads), 0, st, p);
    }
  };
  auto go = [&](auto dc, auto hc) {
    if (p.window > 0) go2(dc, hc, std::true_type{});
    else go2(dc, hc, std::false_type{});
  };
  auto by_hpw = [&](auto dc) {
    if (hpw == 4) go(dc, std::integral_constant<int, 4>{});
    else if (hpw == 2) go(dc, std::integral_constant<int, 2>{});
    else go(dc, std::integral_constant<int, 1>{});
  };
  switch (head_dim) {
    case 32: by_hpw(std::integral_constant<int, 32>{}); break;
    case 64: by_hpw(std::integral_constant<int, 64>{}); break;
    case 256: by_hpw(std::integral_constant<int, 256>{}); break;
    default: by_hpw(std::integral_constant<int, 128>{}); break;
  }
}

}  // namespace

// The streaming kernel for each scale mode (kvq_decode_token.hip,
// kvq_decode_group32.hip, kvq_decode_bf16.hip, kvq_decode_fp8.hip).
void launch_stream_token(int head_dim, int hpw, bool paged, bool append, const DecodeParams& p, dim3 grid,
                         hipStream_t st);
void launch_stream_group32(int head_dim, int hpw, bool paged, bool append, const DecodeParams& p, dim3 grid,
                           hipStream_t st);
void launch_stream_bf16(int head_dim, int hpw, bool paged, bool append, const DecodeParams& p, dim3 grid,
                        hipStream_t st);
void launch_stream_fp8(int head_dim, int hpw, int sm, bool paged, bool append, const DecodeParams& p, dim3 grid,
                       hipStream_t st);

}  // namespace kvq
