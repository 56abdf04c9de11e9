// Chunked-prefill attention on the INT8 KV cache (gfx950 MFMA).
//
// n new queries of sequence b sit at absolute positions L0_b + i and attend to
// the cached tokens, the chunk's own rows included.  Causal masking is aligned
// bottom-right: query i sees keys t <= L0_b + i (abaddon 0.2.0-rc.1
// src/kv_cache_quant_cuda.rs, `forward_attention`, cache_offset = seq_len -
// q_len; combs-models 0.2.2 src/kv.rs, `attend`, keys after the query position
// forbidden).  Scores and the weighted value sum are dense contractions and run
// on v_mfma_f32_32x32x16_f16:
//   * K and V codes become exact f16 values c - 128 (v_perm_b32 puts a code
//     under the f16 exponent of 1024, v_pk_add_f16 subtracts 1152).  Queries
//     are scaled by a power of two into f16 range, exact for bf16 inputs.  The
//     per-token K scale multiplies the fp32 score; the per-token V scale is
//     folded into the exponent of the weight, w_t = 2^(S_t log2 e + log2 sV_t
//     - m), and the normaliser sums w_t / sV_t.  Only the f16 weights are
//     rounded before the fp32 accumulation.
//   * S^T = K Q^T gives each lane one query column; in the 32x32 C layout a
//     lane's 16 token rows are exactly the k-slots the B operand of the
//     second product O^T = V^T P^T needs, so the weights never leave their
//     lanes.  V^T comes out of a row-major LDS tile through ds_read_b64_tr_b8
//     (each lane of a 16-lane group names one 8-byte row piece; lane j gets
//     byte j % 8 of the pieces named by lanes 2b + j / 8, b = 0..7).
//   * one workgroup = 4 waves = 4 (query head, 32-position block) items of
//     one KV head; the 64-token K/V tile is staged once in LDS (double
//     buffered, XOR-swizzled in 8-byte units) and serves all four.  With
//     H / KVH a multiple of 4 the four items share their positions.
//   * the running maximum per query is lazy: accumulators are rescaled only
//     when a score exceeds it by more than 2^8, so weights stay below 2^8.
#include "kvq_internal.hpp"

namespace kvq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kCkWaves = 4;
constexpr int kCkThreads = kCkWaves * kWave;
constexpr int kCkTile = 64;   // tokens per pipeline stage
constexpr int kQBlock = 32;   // query positions per wave
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
  float scale_log2;     // attn_scale * log2(e)
};

// 8-byte unit permutation of a D-byte code row, chosen so that the 32 lanes
// of one K read (32 rows, one unit) and of one V transpose read (8 rows x 4
// units) fall on distinct banks.
template <int D>
__device__ __forceinline__ int swz(int t) {
  if constexpr (D == 128) {
    const int s = (t >> 1) & 15;
    return ((s & 1) << 2) | (((s >> 2) & 1) << 3) | ((s >> 1) & 1) | (((s >> 3) & 1) << 1);
  } else {
    const int s = (t >> 2) & 7;
    return (((s >> 1) & 1) << 2) | ((s & 1) << 1) | ((s >> 2) & 1);
  }
}

// Byte offset of 8-byte unit u of tile row t.
template <int D>
__device__ __forceinline__ int tile_off(int t, int u) {
  return t * D + 8 * (u ^ swz<D>(t));
}

// Eight codes -> eight exact f16 values c - 128.
__device__ __forceinline__ f16x8 codes_f16(uint32_t lo, uint32_t hi) {
  const uint32_t e = 0x64646464u;  // high byte of f16 1024 + c
  uint4 w;
  w.x = __builtin_amdgcn_perm(e, lo, 0x04010400u);
  w.y = __builtin_amdgcn_perm(e, lo, 0x04030402u);
  w.z = __builtin_amdgcn_perm(e, hi, 0x04010400u);
  w.w = __builtin_amdgcn_perm(e, hi, 0x04030402u);
  const f16x2 off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  f16x2 p0 = __builtin_bit_cast(f16x2, w.x) + off;
  f16x2 p1 = __builtin_bit_cast(f16x2, w.y) + off;
  f16x2 p2 = __builtin_bit_cast(f16x2, w.z) + off;
  f16x2 p3 = __builtin_bit_cast(f16x2, w.w) + off;
  f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
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

template <int D, bool PAGED>
__device__ __forceinline__ int64_t row_of(const ChunkParams& p, int b, int g, int t) {
  if constexpr (PAGED) {
    int phys = p.geom.block_table[static_cast<int64_t>(b) * p.geom.max_blocks + (t >> 4)];
    phys = min(max(phys, 0), p.geom.num_pages - 1);
    return (static_cast<int64_t>(phys) * p.geom.kvh + g) * kPageSize + (t & (kPageSize - 1));
  } else {
    return (static_cast<int64_t>(b) * p.geom.kvh + g) * p.geom.max_len + t;
  }
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kCkThreads, 2) void chunk_kernel(ChunkParams p) {
  constexpr int kTileBytes = kCkTile * D;
  constexpr int kChunksPerRow = D / 16;                          // 16-byte pieces
  constexpr int kLoads = kCkTile * kChunksPerRow / kCkThreads;   // per side per thread
  constexpr int kKK = D / 16;                                    // MFMA k-steps for S
  constexpr int kDT = D / 32;                                    // 32-wide d tiles of O
  static_assert(kLoads >= 1, "tile loader");

  __shared__ __attribute__((aligned(16))) uint8_t sm_k[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sm_v[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sm_sk[2][kCkTile];
  __shared__ __attribute__((aligned(16))) float sm_lsv[2][kCkTile];
  __shared__ __attribute__((aligned(16))) float sm_rsv[2][kCkTile];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 31;   // query column of this lane
  const int half = lane >> 5;  // which 8 of each 16 k-slots

  // Consecutive blockIdx land on different XCDs; give each XCD a contiguous
  // range of logical ids so the workgroups of one KV head share an L2.
  int bid = blockIdx.x;
  if ((p.total_wgs & 7) == 0) bid = (bid & 7) * (p.total_wgs >> 3) + (bid >> 3);
  const int wg = bid % p.wgs_per_bg;
  const int bg = bid / p.wgs_per_bg;
  const int g = bg % p.geom.kvh;
  const int b = bg / p.geom.kvh;

  const int cap = capacity(p.geom);
  const int L0 = min(max(p.ctx_lens[b], 0), cap);
  const int Ltot = min(L0 + p.n, cap);   // keys that exist
  const int items = p.hpg * p.nblk;

  auto wave_end = [&](int w) -> int {
    const int it = wg * kCkWaves + w;
    if (it >= items) return 0;
    const int pb = (it / p.hpg) * kQBlock;
    return p.causal ? min(L0 + pb + kQBlock, Ltot) : Ltot;
  };
  const int wg_end = max(max(wave_end(0), wave_end(1)), max(wave_end(2), wave_end(3)));
  const int ntiles = (wg_end + kCkTile - 1) / kCkTile;

  const int item = wg * kCkWaves + wave;
  const bool active = item < items;
  const int head = g * p.hpg + (active ? item % p.hpg : 0);
  const int pos0 = active ? (item / p.hpg) * kQBlock : 0;
  const int my_end = wave_end(wave);
  const int qi = pos0 + col;
  const bool q_ok = active && qi < p.n;

  // ---- query operand: B of S^T = K Q^T (k-slot 8*half + e <-> d = 16kk + 8*half + e)
  f16x8 qop[kKK];
  float cq;
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * p.heads + head) * p.n + (q_ok ? qi : 0)) * D;
    uint4 raw[kKK];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      raw[kk] = q_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {raw[kk].x, raw[kk].y, raw[kk].z, raw[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] & 0xffff0000u)));
      }
    }
    amax = other_half_max(amax);
    int kq = 0;
    if (amax > 0.0f && amax <= 3.0e38f) {
      int ex;
      (void)frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
      kq = min(max(15 - ex, -120), 120);
    }
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const uint32_t w[4] = {raw[kk].x, raw[kk].y, raw[kk].z, raw[kk].w};
      f16x8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 h2 = pack2(ldexpf(__uint_as_float(w[e] << 16), kq), ldexpf(__uint_as_float(w[e] & 0xffff0000u), kq));
        v[2 * e] = h2[0];
        v[2 * e + 1] = h2[1];
      }
      qop[kk] = v;
    }
    cq = ldexpf(p.scale_log2, -kq);
  }

  // ---- tile loader: 16-byte pieces of K and V rows plus per-token scales
  uint4 kreg[kLoads], vreg[kLoads];
  float sreg = 0.0f;
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int id = tid + i * kCkThreads;
      const int r = id / kChunksPerRow;
      const int c = id % kChunksPerRow;
      int t = t0 + r;
      t = t < Ltot ? t : Ltot - 1;
      const int64_t row = row_of<D, PAGED>(p, b, g, t);
      kreg[i] = *reinterpret_cast<const uint4*>(p.k_codes + row * D + 16 * c);
      vreg[i] = *reinterpret_cast<const uint4*>(p.v_codes + row * D + 16 * c);
    }
    if (tid < 2 * kCkTile) {
      const int t = t0 + (tid & (kCkTile - 1));
      if (t < Ltot) {
        const int64_t row = row_of<D, PAGED>(p, b, g, t);
        sreg = tid < kCkTile ? p.k_scales[row] : p.v_scales[row];
      }
    }
  };
  auto store_tile = [&](int buf, int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int id = tid + i * kCkThreads;
      const int r = id / kChunksPerRow;
      const int c = id % kChunksPerRow;
      const int f = swz<D>(r);
      const int off = r * D + 8 * ((2 * c) ^ (f & ~1));
      uint4 kv = kreg[i], vv = vreg[i];
      if (f & 1) {
        kv = make_uint4(kv.z, kv.w, kv.x, kv.y);
        vv = make_uint4(vv.z, vv.w, vv.x, vv.y);
      }
      *reinterpret_cast<uint4*>(&sm_k[buf][off]) = kv;
      *reinterpret_cast<uint4*>(&sm_v[buf][off]) = vv;
    }
    if (tid < 2 * kCkTile) {
      const int tl = tid & (kCkTile - 1);
      const bool ok = t0 + tl < Ltot;
      if (tid < kCkTile) {
        sm_sk[buf][tl] = ok ? sreg : 0.0f;
      } else {
        sm_lsv[buf][tl] = ok ? __builtin_amdgcn_logf(sreg) : -INFINITY;
        sm_rsv[buf][tl] = ok ? 1.0f / sreg : 0.0f;
      }
    }
  };

  // ---- per-lane LDS addresses (loop invariant)
  // K operand: row 32tt + col, unit 2kk + half.
  // V operand (transpose read): lane 16*grp + r names token 16ks + pi(grp/2, r/2)
  // and unit 4dt + 2(grp%2) + r%2, where pi(h, e) = 8(e/4) + 4h + e%4 is the
  // token of k-slot 8h + e in the S^T C layout.
  const int grp = lane >> 4;
  const int r16 = lane & 15;
  const int vtok = 8 * ((r16 >> 1) >> 2) + 4 * (grp >> 1) + ((r16 >> 1) & 3);
  const int vunit = 2 * (grp & 1) + (r16 & 1);

  f32x16 oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[dt] = f32x16{};
  float m_run = kMinusBig;
  float l_run = 0.0f;

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int t0 = it * kCkTile;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(t0 + kCkTile);

    if (active && t0 < my_end) {
      const uint8_t* smk = sm_k[buf];
      const uint8_t* smv = sm_v[buf];
      // S^T tiles: rows = tokens 32tt + (8(r/4) + 4*half + r%4), column = query
      f32x16 s[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        s[tt] = f32x16{};
        const int trow = 32 * tt + col;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          const uint2 c8 = *reinterpret_cast<const uint2*>(smk + tile_off<D>(trow, 2 * kk + half));
          s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(codes_f16(c8.x, c8.y), qop[kk], s[tt], 0, 0, 0);
        }
      }
      // z = S log2 e + log2 sV (per token), masked to -inf where not visible
      const bool diag = p.causal && (t0 + kCkTile - 1 > L0 + pos0);
      const int limit = L0 + qi;
      float z[2][16];
      float zmax = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int tl = 32 * tt + 8 * q4 + 4 * half;
          const float4 sk = *reinterpret_cast<const float4*>(&sm_sk[buf][tl]);
          const float4 lv = *reinterpret_cast<const float4*>(&sm_lsv[buf][tl]);
          const float skv[4] = {sk.x, sk.y, sk.z, sk.w};
          const float lvv[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) z[tt][4 * q4 + e] = fmaf(s[tt][4 * q4 + e], skv[e] * cq, lvv[e]);
        }
      }
      if (diag) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3) > limit) z[tt][r] = -INFINITY;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
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
      // weights, normaliser, and O^T += V^T P^T
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float w[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int tl = 32 * tt + 8 * q4 + 4 * half;
          const float4 rv = *reinterpret_cast<const float4*>(&sm_rsv[buf][tl]);
          const float rvv[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[4 * q4 + e] = __builtin_amdgcn_exp2f(z[tt][4 * q4 + e] - m_run);
            l_run = fmaf(w[4 * q4 + e], rvv[e], l_run);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 pw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 h2 = pack2(w[8 * ks + 2 * e], w[8 * ks + 2 * e + 1]);
            pw[2 * e] = h2[0];
            pw[2 * e + 1] = h2[1];
          }
          const int tok = 32 * tt + 16 * ks + vtok;
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            const v2i c8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (v2i __attribute__((address_space(3)))*)(smv + tile_off<D>(tok, 4 * dt + vunit)));
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                codes_f16(static_cast<uint32_t>(c8.x), static_cast<uint32_t>(c8.y)), pw, oacc[dt], 0, 0, 0);
          }
        }
      }
    }

    if (more) store_tile(buf ^ 1, t0 + kCkTile);
    __syncthreads();
  }

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

}  // namespace

bool chunk_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

size_t chunk_workspace(const kvq_cache&, int, int) { return 0; }

kvq_status launch_chunk(const kvq_cache& c, const uint16_t* q, int n, const int32_t* ctx_lens, int causal,
                        float attn_scale, uint16_t* out, void*, int, hipStream_t stream) {
  if (c.scale_mode != KVQ_SCALE_PER_TOKEN)
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_attention_chunk: group-32 scales are not supported");
  ChunkParams p;
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
  p.causal = causal ? 1 : 0;
  p.scale_log2 = attn_scale * kCkLog2e;
  const int64_t items = static_cast<int64_t>(p.hpg) * p.nblk;
  const int64_t per_bg = (items + kCkWaves - 1) / kCkWaves;
  const int64_t total = per_bg * c.batch * c.num_kv_heads;
  if (total > 0x7fffffffLL) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_attention_chunk: grid too large");
  p.wgs_per_bg = static_cast<int32_t>(per_bg);
  p.total_wgs = static_cast<int32_t>(total);
  const dim3 grid(static_cast<unsigned>(total));
  const bool paged = c.layout == KVQ_LAYOUT_PAGED;
  if (c.head_dim == 128) {
    if (paged) hipLaunchKernelGGL((chunk_kernel<128, true>), grid, dim3(kCkThreads), 0, stream, p);
    else hipLaunchKernelGGL((chunk_kernel<128, false>), grid, dim3(kCkThreads), 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((chunk_kernel<64, true>), grid, dim3(kCkThreads), 0, stream, p);
    else hipLaunchKernelGGL((chunk_kernel<64, false>), grid, dim3(kCkThreads), 0, stream, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_attention_chunk: launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq
