// Chunked-prefill attention on the INT8 KV cache (gfx950 MFMA).
//
// n new queries of sequence b sit at absolute positions L0_b + i and attend to
// the cached tokens, the chunk's own rows included.  Causal masking is aligned
// bottom-right: query i sees keys t <= L0_b + i (abaddon 0.2.0-rc.1
// src/kv_cache_quant_cuda.rs, `forward_attention`, cache_offset = seq_len -
// q_len; combs-models 0.2.2 src/kv.rs, `attend`, keys after the query position
// forbidden).  Scores and the weighted value sum are dense contractions and run
// on v_mfma_f32_32x32x16_f16:
//   * S^T = K Q^T gives each lane one query column; in the 32x32 C layout a
//     lane's 16 token rows are exactly the k-slots the B operand of the
//     second product O^T = V^T P^T needs, so the weights never leave their
//     lanes.
//   * K and V codes are widened once per workgroup, while staging the tile
//     in LDS, to exact f16 values c - 128 (v_perm_b32 puts a code under the
//     f16 exponent of 1024, v_pk_add_f16 subtracts 1152).  V^T comes out of
//     LDS through ds_read_b64_tr_b16: each lane of a 16-lane group names one
//     8-byte row piece (four f16), and lane j gets element j % 4 of the
//     pieces named by lanes j / 4 + 4b, b = 0..3; two such reads give a
//     lane its eight k-slots.
//   * queries are scaled by powers of two into f16 range (exact for bf16
//     inputs): the per-token K scale, the attention scale, log2 e and the
//     workgroup's power of two (set by its largest query) form one staged
//     factor per token, so a score is one FMA: z_t = acc * kc_t + log2 sV_t;
//     a wave whose own queries are much smaller scales them by a larger power
//     of two and brings its scores back to the workgroup's before the FMA.  The V scale rides in
//     the exponent of the weight, w_t = 2^(z_t - m), and the normaliser sums
//     w_t / sV_t.
//   * one workgroup = 8 waves = 8 (query head, 32-position block) items of
//     one KV head, in two groups of four; each 64-token tile is staged once in
//     LDS (four buffers in rotation) and serves all eight.  With H / KVH a
//     multiple of 4 each group's items share their positions.
//   * the groups ping-pong: each wave alternates an MFMA step (the values of
//     the previous tile, S of this one) and a vector step (this tile's
//     softmax), with a workgroup barrier after each; group 1 runs one step
//     behind, so the two waves that share a SIMD always do opposite kinds of
//     work and the matrix cores overlap the exponentials.
//   * the running maximum per query is lazy: accumulators are rescaled only
//     when a score exceeds it by more than 2^8, so weights stay below 2^8.
#include "kvq_internal.hpp"
#include "kvq_quant.hpp"

#include <type_traits>

namespace kvq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kCkWaves = 8;      // two groups of four, one wave of each per SIMD
constexpr int kGroupWaves = 4;
constexpr int kCkThreads = kCkWaves * kWave;
// tokens per tile: 64, or 32 at head dim 256 (four buffers of 64-token
// tiles would not fit the LDS; a 32-token tile at D = 256 carries the MFMA
// work of a 64-token one at D = 128)
constexpr int tile_tokens(int D) { return D > 128 ? 32 : 64; }
constexpr int kCkBufs = 4;      // LDS tile buffers in rotation
constexpr int kQBlock = 32;     // query positions per wave
constexpr float kCkLog2e = 1.4426950408889634f;
constexpr float kCkLazy = 8.0f;
constexpr float kMinusBig = -1.0e30f;  // running-max start: finite, below any score

struct ChunkParams {
  const uint16_t* q;    // [B, H, n, D] bf16
  uint16_t* out;        // [B, H, n, D] bf16
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_scales;
  const float* v_scales;
  const int32_t* ctx_lens;  // [B]
  CacheGeom geom;
  int32_t heads;
  int32_t hpg;          // query heads per KV head
  int32_t n;
  int32_t nblk;         // ceil(n / 32)
  int32_t wgs_per_bg;   // workgroups per (sequence, KV head)
  int32_t total_wgs;
  int32_t causal;
  int32_t window;       // sliding window (0: none): query p sees keys in (p - window, p]
  float scale_log2;     // attn_scale * log2(e)
  // recent-window cache (rwin > 0): the last rwin of each sequence's L0 + n
  // rows are bf16 rows in ring slot position % rcap, staged in the same
  // tiles as the INT8 rows below them
  int32_t rwin;
  int32_t len_cap;      // hint + n when rwin > 0 (ctx_lens clamp to the hint)
  int32_t rcap;
  const uint16_t* rk;   // [B, KVH, rcap, D] bf16
  const uint16_t* rv;
};

// LDS tile geometry for TOK tokens.  K rows hold D f16 values and are padded
// by 16 bytes, so the 16 lanes of one K read (16 consecutive rows, one
// 16-byte unit) fall on distinct banks.  V rows also hold D f16 values (the
// codes are widened while staging), with the padding described below.
// With group-32 scales (G32) a buffer also holds, per token, the ratios of
// consecutive K group scales s_g / s_(g+1) (fp32, groups 0 .. G-2) and the
// f16 ratios s_g / s_max of V.
template <int D, int TOK, bool G32 = false>
struct Tile {
  static constexpr int kKRow = 2 * D + 16;
  static constexpr int kKBytes = TOK * kKRow;
  // V rows hold D f16 values, padded to a stride of 64 mod 256 bytes: the
  // LDS serves a transposed read 32 lanes (four rows x 64 bytes) at a time,
  // and those then cover every bank once
  static constexpr int kVRow = 2 * D + 64;
  static constexpr int kVBytes = TOK * kVRow;
  static constexpr int kNG = D / 32;
  static constexpr int kBytes = kKBytes + kVBytes + 3 * TOK * 4 + (G32 ? (kNG - 1) * TOK * 4 + kNG * TOK * 2 : 0);
  // byte offsets inside one buffer
  static __device__ __forceinline__ int k_off(int t, int u16) { return t * kKRow + 16 * u16; }
  static __device__ __forceinline__ int v_off(int t, int u16) { return kKBytes + t * kVRow + 16 * u16; }
  static constexpr int kKc = kKBytes + kVBytes;
  static constexpr int kLsv = kKc + TOK * 4;
  static constexpr int kRsv = kLsv + TOK * 4;
  static constexpr int kRk = kRsv + TOK * 4;            // G32: fp32 [group][token], K s_g / s_(g+1)
  static constexpr int kRv = kRk + (kNG - 1) * TOK * 4; // G32: f16 [group][token], V s_g / s_max
};

// Four codes -> two f16 pairs holding the exact values c - 128.
__device__ __forceinline__ uint2 codes_exact_f16(uint32_t w) {
  const uint32_t e = 0x64646464u;  // high byte of f16 1024 + c
  const f16x2 off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, w, 0x04010400u)) + off;
  const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, w, 0x04030402u)) + off;
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

__device__ __forceinline__ f16x2 pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_convertvector(v, f16x2);
}

__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max64(float x) {
  x = fmaxf(x, __shfl_xor(x, 1, kWave));
  x = fmaxf(x, __shfl_xor(x, 2, kWave));
  x = fmaxf(x, __shfl_xor(x, 4, kWave));
  x = fmaxf(x, __shfl_xor(x, 8, kWave));
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return other_half_max(x);
}

template <bool PAGED>
__device__ __forceinline__ int64_t row_of(const ChunkParams& p, int b, int g, int t) {
  if constexpr (PAGED) {
    int phys = p.geom.block_table[static_cast<int64_t>(b) * p.geom.max_blocks + (t >> 4)];
    phys = min(max(phys, 0), p.geom.num_pages - 1);
    return (static_cast<int64_t>(phys) * p.geom.kvh + g) * kPageSize + (t & (kPageSize - 1));
  } else {
    return (static_cast<int64_t>(b) * p.geom.kvh + g) * p.geom.max_len + t;
  }
}

// SM: KVQ_SCALE_PER_TOKEN, KVQ_SCALE_PER_TOKEN_BF16 (scales stored as bf16)
// or an FP8 code format (values, no scales); a template argument so that each
// mode keeps its registers.  RING: a hybrid cache whose ring rows join the
// tiles (below).
template <int D, bool PAGED, int SM, bool RING>
__global__ __launch_bounds__(kCkThreads, 1) void chunk_kernel(ChunkParams p) {
  constexpr bool SBF = SM == KVQ_SCALE_PER_TOKEN_BF16;
  constexpr bool FP8 = SM == KVQ_CODES_FP8_E4M3 || SM == KVQ_CODES_FP8_E5M2;
  constexpr bool E5 = SM == KVQ_CODES_FP8_E5M2;
  // group-32: K stays exact f16 c - 128; the score accumulator takes the
  // group scales in Horner form, multiplied per token by s_g / s_(g+1) after
  // group g's k-steps, with the last group's scale in the token's score
  // factor (all fp32).  V is exact c - 128, and each 32-dim output tile (one
  // group) weights its tokens by s_g / s_max
  constexpr bool G32 = SM == KVQ_SCALE_GROUP32;
  constexpr int NG = D / 32;
  constexpr int kCkTile = tile_tokens(D);
  using TL = Tile<D, kCkTile, G32>;
  constexpr int kTT = kCkTile / 32;                        // 32-token S tiles per tile
  constexpr int kChunksPerRow = D / 16;                    // 16-code pieces per row
  constexpr int kChunks = kCkTile * kChunksPerRow;         // per side per tile
  constexpr int kLoads = (2 * kChunks + kCkThreads - 1) / kCkThreads;  // pieces per thread
  constexpr int kKK = D / 16;                              // MFMA k-steps for S
  constexpr int kDT = D / 32;                              // 32-wide d tiles of O

  __shared__ __attribute__((aligned(16))) uint8_t smem[kCkBufs * TL::kBytes];
  __shared__ float sm_qmax[kCkWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / kGroupWaves;   // 0: leads, 1: one phase behind
  const int col = lane & 31;            // query column of this lane
  const int half = lane >> 5;           // which 8 of each 16 k-slots

  // Consecutive blockIdx land on different XCDs; give each XCD a contiguous
  // range of logical ids so the workgroups of one KV head share an L2.
  int bid = blockIdx.x;
  if ((p.total_wgs & 7) == 0) bid = (bid & 7) * (p.total_wgs >> 3) + (bid >> 3);
  const int wg = bid % p.wgs_per_bg;
  const int bg = bid / p.wgs_per_bg;
  const int g = bg % p.geom.kvh;
  const int b = bg / p.geom.kvh;

  const int cap = RING ? min(capacity(p.geom), p.len_cap) : capacity(p.geom);
  const int L0 = min(max(p.ctx_lens[b], 0), RING ? cap - p.n : cap);
  const int Ltot = min(L0 + p.n, cap);         // keys that exist
  const int L8 = RING ? max(Ltot - p.rwin, 0) : Ltot;  // a hybrid cache's ring rows start here
  const int64_t ring0 = (static_cast<int64_t>(b) * p.geom.kvh + g) * p.rcap;
  const int items = p.hpg * p.nblk;

  int wg_end = 0;
#pragma unroll
  for (int w = 0; w < kCkWaves; ++w) {
    const int it = wg * kCkWaves + w;
    if (it < items) {
      const int pb = (it / p.hpg) * kQBlock;
      wg_end = max(wg_end, p.causal ? min(L0 + pb + kQBlock, Ltot) : Ltot);
    }
  }
  // With a sliding window the tiles start at the lowest key any of the
  // workgroup's queries sees (combs-models kv.rs `attend`: keys at or below
  // p - window are masked), rounded down to a tile.
  int wg_lo = 0;
  if (p.window > 0) {
    wg_lo = wg_end;
#pragma unroll
    for (int w = 0; w < kCkWaves; ++w) {
      const int it = wg * kCkWaves + w;
      if (it < items) wg_lo = min(wg_lo, L0 + (it / p.hpg) * kQBlock - p.window + 1);
    }
    wg_lo = max(wg_lo, 0);
  }
  const int tbase = (wg_lo / kCkTile) * kCkTile;  // token offset of tile 0
  const int ntiles = max((wg_end - tbase + kCkTile - 1) / kCkTile, 0);

  const int item = wg * kCkWaves + wave;
  const bool active = item < items;
  const int head = g * p.hpg + (active ? item % p.hpg : 0);
  const int pos0 = active ? (item / p.hpg) * kQBlock : 0;
  const int qi = pos0 + col;
  const bool q_ok = active && qi < p.n;

  // ---- queries: each wave's largest magnitude (the powers of two are set below)
  uint4 qraw[kKK];
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * p.heads + head) * p.n + (q_ok ? qi : 0)) * D;
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qraw[kk] = q_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {qraw[kk].x, qraw[kk].y, qraw[kk].z, qraw[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] & 0xffff0000u)));
      }
    }
    amax = wave_max64(amax);
    if (lane == 0) sm_qmax[wave] = amax;
  }

  // ---- tile loader: piece j of a tile (j < kChunks: K, else V) is held by
  // thread j % kCkThreads; threads 0..2*kCkTile-1 also hold the per-token
  // scales (first half K, second half V)
  const bool ld_s = tid < 2 * kCkTile;
  uint4 lreg[kLoads];
  uint32_t sreg = 0u;  // scale word as loaded, decoded when the tile is stored
  float greg[G32 ? NG : 1];  // group-32: the token's group scales as loaded
  static_assert(!RING || 2 * kChunks == kLoads * kCkThreads, "ring pieces: every thread holds whole pieces");
  // the clamped key of piece id of the tile at t0 (row 0 stands in when no key exists)
  auto piece_key = [&](int t0, int id) {
    const int t = t0 + id / kChunksPerRow;
    return max(t < Ltot ? t : Ltot - 1, 0);
  };
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = tid + i * kCkThreads;
      if (j < 2 * kChunks) {
        const bool kside = j < kChunks;
        const int id = kside ? j : j - kChunks;
        const int64_t row = row_of<PAGED>(p, b, g, piece_key(t0, id));
        lreg[i] = *reinterpret_cast<const uint4*>((kside ? p.k_codes : p.v_codes) + row * D + 16 * (id % kChunksPerRow));
      }
    }
    if (ld_s && !FP8) {
      const int t = t0 + (tid & (kCkTile - 1));
      if (t < (RING ? L8 : Ltot)) {
        const int64_t row = row_of<PAGED>(p, b, g, t);
        if constexpr (G32) {
          const float* gs = (tid < kCkTile ? p.k_scales : p.v_scales) + row * NG;
          if constexpr (NG == 4) {
            const float4 v = *reinterpret_cast<const float4*>(gs);
            greg[0] = v.x; greg[1] = v.y; greg[2] = v.z; greg[3] = v.w;
          } else {
#pragma unroll
            for (int k = 0; k < NG; ++k) greg[k] = gs[k];
          }
        } else {
          sreg = scale_word(tid < kCkTile ? p.k_scales : p.v_scales, row, SBF);
        }
      }
    }
  };
  auto store_tile = [&](uint8_t* buf, int t0, float kfac) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = tid + i * kCkThreads;
      if (j < 2 * kChunks) {  // K or V: 16 codes -> 16 exact f16 values = units 2c and 2c + 1
        const bool kside = j < kChunks;
        const int id = kside ? j : j - kChunks;
        const int r = id / kChunksPerRow, c = id % kChunksPerRow;
        uint2 k0, k1, k2, k3;
        if constexpr (FP8) {  // the codes' own values
          k0 = make_uint2(fp8_pair_k<E5, false>(lreg[i].x), fp8_pair_k<E5, true>(lreg[i].x));
          k1 = make_uint2(fp8_pair_k<E5, false>(lreg[i].y), fp8_pair_k<E5, true>(lreg[i].y));
          k2 = make_uint2(fp8_pair_k<E5, false>(lreg[i].z), fp8_pair_k<E5, true>(lreg[i].z));
          k3 = make_uint2(fp8_pair_k<E5, false>(lreg[i].w), fp8_pair_k<E5, true>(lreg[i].w));
        } else {
          k0 = codes_exact_f16(lreg[i].x);
          k1 = codes_exact_f16(lreg[i].y);
          k2 = codes_exact_f16(lreg[i].z);
          k3 = codes_exact_f16(lreg[i].w);
        }
        uint8_t* dst = buf + (kside ? TL::k_off(r, 2 * c) : TL::v_off(r, 2 * c));
        *reinterpret_cast<uint4*>(dst) = make_uint4(k0.x, k0.y, k1.x, k1.y);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(k2.x, k2.y, k3.x, k3.y);
      }
    }
    if (ld_s && !(RING && t0 + (tid & (kCkTile - 1)) >= L8 && t0 + (tid & (kCkTile - 1)) < Ltot)) {
      // (a ring row's factors are written by its first piece's thread above)
      const int tl = tid & (kCkTile - 1);
      const bool ok = t0 + tl < Ltot;
      // which half of the word holds a bf16 scale: the parity of the row
      // (page rows start even, so in the paged layout the token's parity)
      const int64_t srow = PAGED ? static_cast<int64_t>(t0 + tl)
                                 : (static_cast<int64_t>(b) * p.geom.kvh + g) * p.geom.max_len + t0 + tl;
      float sv = FP8 ? 1.0f : scale_value(sreg, scale_sel(srow, SBF));
      if constexpr (G32) {
        if (tid < kCkTile) {
          // K: consecutive group ratios; the last group's scale is the factor
          float* rk = reinterpret_cast<float*>(buf + TL::kRk);
#pragma unroll
          for (int k = 0; k + 1 < NG; ++k) rk[k * kCkTile + tl] = ok ? greg[k] / greg[k + 1] : 1.0f;
          sv = greg[NG - 1];
        } else {
          // V: the token's largest group scale, and each group's ratio to it
          sv = greg[0];
#pragma unroll
          for (int k = 1; k < NG; ++k) sv = fmaxf(sv, greg[k]);
          _Float16* rv = reinterpret_cast<_Float16*>(buf + TL::kRv);
#pragma unroll
          for (int k = 0; k < NG; ++k) rv[k * kCkTile + tl] = static_cast<_Float16>(ok ? greg[k] / sv : 0.0f);
        }
      }
      if (tid < kCkTile) {
        reinterpret_cast<float*>(buf + TL::kKc)[tl] = ok ? sv * kfac : 0.0f;
      } else {
        reinterpret_cast<float*>(buf + TL::kLsv)[tl] = ok ? __builtin_amdgcn_logf(sv) : -INFINITY;
        reinterpret_cast<float*>(buf + TL::kRsv)[tl] = ok ? 1.0f / sv : 0.0f;
      }
    }
  };
  // A hybrid cache's ring rows, in the tiles that hold any: store_tile has
  // staged the INT8 storage at their positions; each thread overwrites the
  // pieces it stored there (so its own later writes win) with the ring row
  // converted to f16 values x 2^sh, sh set by the row's largest |x| (a
  // reduction over the row's pieces, which consecutive threads hold) so
  // that it lands in [2^14, 2^15): exact for every element within 2^28 of
  // that largest.  The row's per-token factors carry 2^-sh, as an INT8
  // row's carry its scale (store_tile leaves them to this step).  Kept out
  // of the loader so that the tiles without ring rows run the plain code.
  auto ring_fixup = [&](uint8_t* buf, int t0, float kfac) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = tid + i * kCkThreads;
      const bool kside = j < kChunks;
      const int id = kside ? j : j - kChunks;
      const int r = id / kChunksPerRow, c = id % kChunksPerRow;
      const int t = piece_key(t0, id);
      const bool ring = t >= L8;
      const uint4* src =
          reinterpret_cast<const uint4*>((kside ? p.rk : p.rv) + (ring0 + t % p.rcap) * D + 16 * c);
      const uint4 a0 = src[0], a1 = src[1];
      const uint32_t wv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float x[16];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[2 * e] = __uint_as_float(wv[e] << 16);
        x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        m = fmaxf(m, fmaxf(fabsf(x[2 * e]), fabsf(x[2 * e + 1])));
      }
      if (!ring) m = 0.0f;
#pragma unroll
      for (int off = 1; off < kChunksPerRow; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
      const int sh = m > 0.0f && m <= 3.4e38f ? min(max(14 - ilogbf(m), -120), 120) : 0;
      if (ring) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = __builtin_bit_cast(uint32_t, pack2(ldexpf(x[2 * e], sh), ldexpf(x[2 * e + 1], sh)));
        uint8_t* dst = buf + (kside ? TL::k_off(r, 2 * c) : TL::v_off(r, 2 * c));
        *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(h[4], h[5], h[6], h[7]);
        if (c == 0 && t0 + r < Ltot) {
          if (kside) {
            reinterpret_cast<float*>(buf + TL::kKc)[r] = ldexpf(kfac, -sh);
            if constexpr (G32) {
              float* rk = reinterpret_cast<float*>(buf + TL::kRk);
#pragma unroll
              for (int k = 0; k + 1 < NG; ++k) rk[k * kCkTile + r] = 1.0f;
            }
          } else {
            reinterpret_cast<float*>(buf + TL::kLsv)[r] = static_cast<float>(-sh);
            reinterpret_cast<float*>(buf + TL::kRsv)[r] = ldexpf(1.0f, sh);
            if constexpr (G32) {
              _Float16* rv = reinterpret_cast<_Float16*>(buf + TL::kRv);
#pragma unroll
              for (int k = 0; k < NG; ++k) rv[k * kCkTile + r] = static_cast<_Float16>(1.0f);
            }
          }
        }
      }
    }
  };
  // stage tile t0 into buf: the loaded pieces, then (hybrid caches) its ring rows
  auto stage_tile = [&](uint8_t* buf, int t0, float kfac) {
    store_tile(buf, t0, kfac);
    if constexpr (RING) {
      if (t0 + kCkTile > L8) ring_fixup(buf, t0, kfac);
    }
  };

  {
    // the first MFMA step takes the last buffer's values times all-zero
    // weights before anything is staged there; f16 bits left in LDS could be
    // NaN or inf (group-32: the V group ratios too), and 0 * NaN is NaN, so
    // those values start as zeros
    uint8_t* bz = smem + (kCkBufs - 1) * TL::kBytes + TL::kKBytes;
    for (int i = tid * 16; i < TL::kVBytes; i += kCkThreads * 16)
      *reinterpret_cast<uint4*>(bz + i) = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (G32) {
      uint8_t* br = smem + (kCkBufs - 1) * TL::kBytes + TL::kRv;
      for (int i = tid * 16; i < TL::kNG * kCkTile * 2; i += kCkThreads * 16)
        *reinterpret_cast<uint4*>(br + i) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  load_tile(tbase);
  __syncthreads();  // sm_qmax (and the cleared values)

  // The staged K factor carries the workgroup's power of two 2^-kq (set by
  // its largest query); each wave scales its own queries by 2^kqw (set by
  // its own largest), so a head much smaller than another head of the
  // workgroup keeps its bits instead of falling into f16 subnormals, and
  // multiplies its scores by 2^(kq - kqw) <= 1 before the K factor (a
  // uniform branch, not taken when the two agree).
  auto pow2_for = [](float amax, int dflt) {
    if (!(amax > 0.0f && amax <= 3.0e38f)) return dflt;
    int ex;
    (void)frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
    return min(max(15 - ex, -120), 120);
  };
  int kq = 0;
  {
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < kCkWaves; ++w) amax = fmaxf(amax, sm_qmax[w]);
    kq = pow2_for(amax, 0);
  }
  const int kqw = __builtin_amdgcn_readfirstlane(pow2_for(sm_qmax[wave], kq));
  const float qcorr = ldexpf(1.0f, kq - kqw);
  const float kfac = ldexpf(p.scale_log2, -kq);
  f16x8 qop[kKK];  // B of S^T = K Q^T: k-slot 8*half + e <-> d = 16kk + 8*half + e
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    const uint32_t w[4] = {qraw[kk].x, qraw[kk].y, qraw[kk].z, qraw[kk].w};
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 h2 = pack2(ldexpf(__uint_as_float(w[e] << 16), kqw), ldexpf(__uint_as_float(w[e] & 0xffff0000u), kqw));
      v[2 * e] = h2[0];
      v[2 * e + 1] = h2[1];
    }
    qop[kk] = v;
  }

  // Prologue: tiles 0 and 1 in LDS, tile 2 in flight.
  stage_tile(smem, tbase, kfac);
  if (ntiles > 1) {
    load_tile(tbase + kCkTile);
    stage_tile(smem + TL::kBytes, tbase + kCkTile, kfac);
  }
  if (ntiles > 2) load_tile(tbase + 2 * kCkTile);
  __syncthreads();

  // V transpose reads: lane 16G + n names token 16ks + 4(G/2) + n/4 (the
  // second read 8 further) and f16 column 16(G%2) + 4(n%4) of the d tile, so
  // it receives column d = lane % 32 at k-slots 8h + e, h = lane / 32, whose
  // tokens pi(h, e) = 8(e/4) + 4h + e%4 are those of the S^T C layout.
  const int vtok = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[dt] = f32x16{};
  float m_run = kMinusBig;
  float l_run = 0.0f;   // sum of w / sV over this lane's tokens
  f32x16 s[kTT];        // S^T of the tile whose softmax comes next
  f16x8 pw[kTT][2];     // weights of the tile whose values come next
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt) {
    s[tt] = f32x16{};
    pw[tt][0] = f16x8{};
    pw[tt][1] = f16x8{};
  }

  // Ping-pong.  Each wave runs, per tile t, an MFMA step (the values of tile
  // t - 1 and S for tile t) and a vector step (the softmax of tile t), each
  // closed by a workgroup barrier.  Group 1 starts one barrier later, so the
  // two waves sharing a SIMD always run opposite kinds of work.  In global
  // phase 2t + 1 (group 0's vector step, group 1's MFMA step) the loader
  // stores tile t + 2 and fetches tile t + 3: tile t + 2's buffer last held
  // tile t - 2, whose last reader (group 1's values, phase 2t - 1) is past.
  // Waves past their last visible key still run: every key they see there is
  // masked, so nothing is added.
  auto mfma_step = [&](int t) {
    __builtin_amdgcn_s_setprio(1);
    {  // values of tile t - 1 (all-zero weights before the first tile)
      const uint8_t* bv = smem + ((t + kCkBufs - 1) % kCkBufs) * TL::kBytes;
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int tok = 32 * tt + 16 * ks + vtok;
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            const uint8_t* va = bv + TL::kKBytes + tok * TL::kVRow + 2 * (32 * dt + vcol);
            const f16x4 a0 = __builtin_bit_cast(
                f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)va));
            const f16x4 a1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                           (v4s __attribute__((address_space(3)))*)(va + 8 * TL::kVRow)));
            const f16x8 a8 = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            if constexpr (G32) {
              // tile dt is group dt: the weights of its tokens times s_g / s_max
              const _Float16* rv = reinterpret_cast<const _Float16*>(bv + TL::kRv) + dt * kCkTile + 32 * tt + 16 * ks +
                                   4 * half;
              const f16x4 r0 = *reinterpret_cast<const f16x4*>(rv);
              const f16x4 r1 = *reinterpret_cast<const f16x4*>(rv + 8);
              const f16x8 r8 = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, pw[tt][ks] * r8, oacc[dt], 0, 0, 0);
            } else {
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, pw[tt][ks], oacc[dt], 0, 0, 0);
            }
          }
        }
      }
    }
    {  // S^T of tile t: rows = tokens 32tt + 8(r/4) + 4*half + r%4, column = query
      const uint8_t* bk = smem + (t % kCkBufs) * TL::kBytes;
      f16x8 ka[kTT];
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
        s[tt] = f32x16{};
        ka[tt] = *reinterpret_cast<const f16x8*>(bk + TL::k_off(32 * tt + col, half));
      }
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        f16x8 na[kTT];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
          na[tt] = kk + 1 < kKK ? *reinterpret_cast<const f16x8*>(bk + TL::k_off(32 * tt + col, 2 * (kk + 1) + half))
                                : ka[tt];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) {
          s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[tt], qop[kk], s[tt], 0, 0, 0);
          ka[tt] = na[tt];
        }
        if constexpr (G32) {
          if (kk % 2 == 1 && kk + 1 < kKK) {  // group kk / 2 complete: Horner step
            const float* rk = reinterpret_cast<const float*>(bk + TL::kRk) + (kk / 2) * kCkTile;
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const float4 f = *reinterpret_cast<const float4*>(rk + 32 * tt + 8 * q4 + 4 * half);
                s[tt][4 * q4 + 0] *= f.x;
                s[tt][4 * q4 + 1] *= f.y;
                s[tt][4 * q4 + 2] *= f.z;
                s[tt][4 * q4 + 3] *= f.w;
              }
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax_step = [&](int t) {
    const int t0 = tbase + t * kCkTile;
    const uint8_t* bc = smem + (t % kCkBufs) * TL::kBytes;
    const float* kc = reinterpret_cast<const float*>(bc + TL::kKc);
    const float* lsv = reinterpret_cast<const float*>(bc + TL::kLsv);
    const float* rsv = reinterpret_cast<const float*>(bc + TL::kRsv);
    if (kqw != kq) {  // this wave's queries carry a larger power of two than the K factor expects
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) s[tt] *= qcorr;
    }
    float z[kTT][16];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int tl = 32 * tt + 8 * q4 + 4 * half;
        const float4 a = *reinterpret_cast<const float4*>(kc + tl);
        const float4 c = *reinterpret_cast<const float4*>(lsv + tl);
        z[tt][4 * q4 + 0] = fmaf(s[tt][4 * q4 + 0], a.x, c.x);
        z[tt][4 * q4 + 1] = fmaf(s[tt][4 * q4 + 1], a.y, c.y);
        z[tt][4 * q4 + 2] = fmaf(s[tt][4 * q4 + 2], a.z, c.z);
        z[tt][4 * q4 + 3] = fmaf(s[tt][4 * q4 + 3], a.w, c.w);
      }
    }
    if (p.causal && t0 + kCkTile - 1 > L0 + pos0) {  // tile reaches the diagonal
      const int limit = L0 + qi - t0;
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tt + 8 * (r >> 2) + 4 * half + (r & 3) > limit) z[tt][r] = -INFINITY;
    }
    if (p.window > 0 && t0 < L0 + pos0 + kQBlock - p.window) {  // tile reaches below a window
      const int lower = L0 + qi - p.window + 1 - t0;               // first visible key of the tile
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tt + 8 * (r >> 2) + 4 * half + (r & 3) < lower) z[tt][r] = -INFINITY;
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) zmax = fmaxf(zmax, z[tt][r]);
    zmax = other_half_max(zmax);
    const bool need = zmax > m_run + kCkLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? zmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= alpha;
    }
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float4 r0 = *reinterpret_cast<const float4*>(rsv + 32 * tt + 16 * ks + 4 * half);
        const float4 r1 = *reinterpret_cast<const float4*>(rsv + 32 * tt + 16 * ks + 8 + 4 * half);
        const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[e] = __builtin_amdgcn_exp2f(z[tt][8 * ks + e] - m_run);
          l_run = fmaf(w[e], rv[e], l_run);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 h2 = pack2(w[2 * e], w[2 * e + 1]);
          pw[tt][ks][2 * e] = h2[0];
          pw[tt][ks][2 * e + 1] = h2[1];
        }
      }
    }
  };
  auto loader_step = [&](int t) {
    if (t + 2 < ntiles) stage_tile(smem + ((t + 2) % kCkBufs) * TL::kBytes, tbase + (t + 2) * kCkTile, kfac);
    if (t + 3 < ntiles) load_tile(tbase + (t + 3) * kCkTile);
  };

  // Where each group's share of the loader work goes.  Both groups may store
  // tile t + 2 in their own MFMA phase (group 0 in phase 2t, group 1 in
  // 2t + 1): its buffer last held tile t - 2, whose last reader, group 1's
  // values of tile t - 2, ran in phase 2t - 1.  Doing so frees registers the
  // ring fix-up and head dim 256 need; elsewhere group 0 stores in its vector
  // phase, which measured no different.
  constexpr bool kLoadInMfma = RING || D == 256;
  if (grp == 1) __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    mfma_step(t);
    if (kLoadInMfma || grp == 1) loader_step(t);
    __syncthreads();
    softmax_step(t);
    if (!kLoadInMfma && grp == 0) loader_step(t);
    __syncthreads();
  }
  mfma_step(ntiles);  // values of the last tile (its S product is unused)
  __syncthreads();
  if (grp == 0) __syncthreads();

  // ---- normalise and store: lane holds query qi, d = 32dt + 8(r/4) + 4*half + r%4
  if (!q_ok) return;
  const float l_tot = other_half_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = p.out + ((static_cast<int64_t>(b) * p.heads + head) * p.n + qi) * D;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      ushort4 o;
      o.x = f32_to_bf16_rne(oacc[dt][4 * q4 + 0] * inv);
      o.y = f32_to_bf16_rne(oacc[dt][4 * q4 + 1] * inv);
      o.z = f32_to_bf16_rne(oacc[dt][4 * q4 + 2] * inv);
      o.w = f32_to_bf16_rne(oacc[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<ushort4*>(orow + 32 * dt + 8 * q4 + 4 * half) = o;
    }
  }
}

template <int D, int SM>
void launch_chunk_sm(bool paged, bool ring, dim3 grid, hipStream_t stream, const ChunkParams& p) {
  constexpr bool FP8 = SM == KVQ_CODES_FP8_E4M3 || SM == KVQ_CODES_FP8_E5M2;
  if constexpr (!FP8 && D != 256) {  // hybrid caches: INT8 codes, head dims 64 and 128
    if (ring) {
      if (paged) hipLaunchKernelGGL((chunk_kernel<D, true, SM, true>), grid, dim3(kCkThreads), 0, stream, p);
      else hipLaunchKernelGGL((chunk_kernel<D, false, SM, true>), grid, dim3(kCkThreads), 0, stream, p);
      return;
    }
  }
  if (paged) hipLaunchKernelGGL((chunk_kernel<D, true, SM, false>), grid, dim3(kCkThreads), 0, stream, p);
  else hipLaunchKernelGGL((chunk_kernel<D, false, SM, false>), grid, dim3(kCkThreads), 0, stream, p);
}

template <int D>
void launch_chunk_d(bool paged, bool ring, int sm, dim3 grid, hipStream_t stream, const ChunkParams& p) {
  switch (sm) {
    case KVQ_SCALE_PER_TOKEN_BF16: launch_chunk_sm<D, KVQ_SCALE_PER_TOKEN_BF16>(paged, ring, grid, stream, p); break;
    case KVQ_CODES_FP8_E4M3: launch_chunk_sm<D, KVQ_CODES_FP8_E4M3>(paged, ring, grid, stream, p); break;
    case KVQ_CODES_FP8_E5M2: launch_chunk_sm<D, KVQ_CODES_FP8_E5M2>(paged, ring, grid, stream, p); break;
    case KVQ_SCALE_GROUP32: launch_chunk_sm<D, KVQ_SCALE_GROUP32>(paged, ring, grid, stream, p); break;
    default: launch_chunk_sm<D, KVQ_SCALE_PER_TOKEN>(paged, ring, grid, stream, p); break;
  }
}

}  // namespace

bool chunk_supported(int head_dim) { return head_dim == 64 || head_dim == 128 || head_dim == 256; }

size_t chunk_workspace(const kvq_cache&, int, int) { return 0; }

kvq_status launch_chunk(const kvq_cache& c, const uint16_t* q, int n, const int32_t* ctx_lens, int causal,
                        float attn_scale, uint16_t* out, void*, int max_ctx_len, hipStream_t stream, int window,
                        const RecentGeom* ring) {
  ChunkParams p{};
  p.q = q;
  p.out = out;
  p.k_codes = c.k_codes;
  p.v_codes = c.v_codes;
  p.k_scales = c.k_scales;
  p.v_scales = c.v_scales;
  p.ctx_lens = ctx_lens;
  p.geom = geom_of(c);
  p.heads = c.num_heads;
  p.hpg = c.num_heads / c.num_kv_heads;
  p.n = n;
  p.nblk = (n + kQBlock - 1) / kQBlock;
  p.causal = causal || window > 0 ? 1 : 0;
  p.window = window > 0 ? window : 0;
  p.scale_log2 = attn_scale * kCkLog2e;
  const bool hybrid = ring != nullptr && ring->window > 0;
  if (hybrid) {
    if (c.head_dim != 64 && c.head_dim != 128)
      return fail(KVQ_ERR_UNSUPPORTED, "kvq_attention_chunk_recent: the MFMA path takes head dims 64 and 128");
    p.rwin = ring->window;
    p.len_cap = max_ctx_len + n;
    p.rcap = ring->cap;
    p.rk = ring->k;
    p.rv = ring->v;
  }
  const int64_t items = static_cast<int64_t>(p.hpg) * p.nblk;
  const int64_t per_bg = (items + kCkWaves - 1) / kCkWaves;
  const int64_t total = per_bg * c.batch * c.num_kv_heads;
  if (total > 0x7fffffffLL) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_chunk: grid too large");
  p.wgs_per_bg = static_cast<int32_t>(per_bg);
  p.total_wgs = static_cast<int32_t>(total);
  const dim3 grid(static_cast<unsigned>(total));
  const bool paged = c.layout == KVQ_LAYOUT_PAGED;
  if (c.head_dim == 128) launch_chunk_d<128>(paged, hybrid, kernel_scale_mode(c), grid, stream, p);
  else if (c.head_dim == 256) launch_chunk_d<256>(paged, hybrid, kernel_scale_mode(c), grid, stream, p);
  else launch_chunk_d<64>(paged, hybrid, kernel_scale_mode(c), grid, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_chunk: launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq
