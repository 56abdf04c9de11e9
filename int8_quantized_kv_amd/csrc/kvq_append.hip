// Quantize-on-append and dequantization kernels.
//
// One wave64 per token row (b, kv head, token) of K or V: the lanes load the
// row with one vector load each, reduce |x| to the row (or 32-element group)
// maximum across lanes, and emit codes with a correctly rounded fp32
// division and round-half-away-from-zero (abaddon 0.2.0-rc.1
// src/kv_cache_quant_cuda.rs, `CudaQuantizedKvCache::quantize_tensor`;
// group-32 from combs-models 0.2.2 src/kv.rs, `kv_quantize`).  The maximum is
// exact, so the reduction order cannot change a code.
#include "kvq_internal.hpp"
#include "kvq_quant.hpp"

namespace kvq {
namespace {

// Modes with a recent window (abaddon 0.2.0-rc.1 kv_cache_quant_cuda.rs,
// `OptimizedQuantizedKvCache::append`): kRows places new rows (below the new
// window: quantized from their bf16 value; inside it: bf16 in the ring);
// kEvict quantizes the ring rows that leave the window, and runs first.
enum AppendMode : int32_t { kPlain = 0, kRows = 1, kEvict = 2 };

struct AppendParams {
  const void* src[2];        // K, V new rows [B, KVH, n_new, D]
  uint8_t* codes[2];
  float* scales[2];
  uint16_t* ring[2];         // recent window: bf16 [B, KVH, rcap, D]
  const int32_t* start_pos;  // [B]; with pos_from_lens, seq_lens [B]
  CacheGeom geom;
  int32_t batch, n, head_dim, groups;  // n: rows per (sequence, KV head) this launch covers
  int32_t n_new;                       // rows appended per sequence
  int32_t rows_per_side;               // B * KVH * n
  int32_t pos_from_lens;               // 1: the row goes to position seq_lens[b] - 1
  int32_t in_bf16;
  int32_t mode;                        // AppendMode
  int32_t rwin, rcap;                  // recent window and ring slots
  int32_t scale_bf16;                  // per-token scales stored as bf16
  int32_t fp8;                         // FP8 codes: 1 E4M3, 2 E5M2 (no scales); 0 INT8
  int32_t block;                       // block scales: 1 per head, 2 per channel (the block pass
                                       // writes every row below the window); 0 per row
  int32_t nblk;                        // block pass: blocks per (sequence, KV head) this launch covers
};

// Stores this lane's EPL values of a row as bf16 (nearest even).
template <int EPL>
__device__ __forceinline__ void store_lane_bf16(uint16_t* row, int lane, const float (&x)[EPL]) {
  uint16_t* out = row + lane * EPL;
  if constexpr (EPL == 1) {
    out[0] = f32_to_bf16_rne(x[0]);
  } else if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = f32_to_bf16_rne(x[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(x[1])) << 16);
  } else {
    uint2 v;
    v.x = f32_to_bf16_rne(x[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(x[1])) << 16);
    v.y = f32_to_bf16_rne(x[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(x[3])) << 16);
    *reinterpret_cast<uint2*>(out) = v;
  }
}

// One wave per row; EPL elements per lane (row_epl(D)); GROUP32: one scale
// per 32 elements (32/EPL lanes) instead of one per row.
template <int EPL, bool GROUP32>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= 2 * p.rows_per_side) return;
  const int side = r >= p.rows_per_side ? 1 : 0;
  const int row = r - side * p.rows_per_side;
  const int i = row % p.n;
  const int bh = row / p.n;
  const int h = bh % p.geom.kvh;
  const int b = bh / p.geom.kvh;
  const int D = p.head_dim;
  const bool on = lane < D / EPL;
  float x[EPL];
  int pos;
  // first position this call appends (with pos_from_lens the array holds
  // lengths, and the one new row sits at length - 1)
  const int start = p.pos_from_lens ? p.start_pos[b] - 1 : p.start_pos[b];
  if (p.mode == kEvict) {
    // ring row q = start - W + i leaves the window (i < min(n_new, W))
    pos = start - p.rwin + i;
    if (pos < 0) return;
    const uint16_t* src = p.ring[side] + (static_cast<int64_t>(bh) * p.rcap + pos % p.rcap) * D;
    load_row_values<EPL>(src, lane, on, true, x);
  } else {
    pos = start + i;
    const size_t esize = p.in_bf16 ? 2 : 4;
    load_row_values<EPL>(static_cast<const char*>(p.src[side]) + static_cast<int64_t>(row) * D * esize, lane, on,
                         p.in_bf16 != 0, x);
    if (p.mode == kRows) {
      // rows enter as bf16 values; those inside the new window go to the ring
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = bf16_to_f32(f32_to_bf16_rne(x[e]));
      if (pos >= start + p.n_new - p.rwin) {
        if (pos < 0) return;
        if (on) store_lane_bf16<EPL>(p.ring[side] + (static_cast<int64_t>(bh) * p.rcap + pos % p.rcap) * D, lane, x);
        return;
      }
      if (p.block) return;  // below the window: written by the block pass
    }
  }
  const int64_t dst = cache_row(p.geom, b, h, pos);
  if (dst < 0) return;  // outside the cache: not written

  float s = 0.0f;
  uint32_t packed;
  if (p.fp8 == 2) packed = fp8_encode_lane<EPL, true>(x);
  else if (p.fp8 == 1) packed = fp8_encode_lane<EPL, false>(x);
  else packed = quantize_lane<EPL, GROUP32>(x, s);  // (p.fp8 is uniform: every lane joins the reduction)
  if (on) {
    store_lane_codes<EPL>(p.codes[side] + dst * D, lane, packed);
    if (p.fp8) return;
    constexpr int kGroupLanes = 32 / EPL;
    float* sc = p.scales[side] + dst * p.groups;
    if (GROUP32) {
      if ((lane % kGroupLanes) == 0) sc[lane / kGroupLanes] = s;
    } else if (lane == 0) {
      store_scale(p.scales[side], dst, s, p.scale_bf16 != 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Block scales on a hybrid cache (abaddon kv_cache_quant_cuda.rs,
// `quantize_with_granularity`, PerHead / PerChannel, over position-aligned
// blocks of kBlockRows rows): block j of a sequence and KV head is quantized
// by the append after which its first row has left the window, i.e. when
// 16j lies in [start - W, L' - W) for this append's first position `start`
// and new length L'.  Its rows are then all present (W >= 15): rows below
// `start` in their ring slots, the others in this append's input (rounded
// to bf16, as every row entering a hybrid cache is).  One wave per (side,
// sequence, KV head, block); lane l holds element indices l, l + 64, ... of
// all 16 rows.  The maximum is exact, so the codes follow the per-token
// quantizer's steps over the block's reduction set: every element of the
// block (per head) or each element index across the 16 rows (per channel).
// Runs before the row pass, which overwrites ring slots.
// ---------------------------------------------------------------------------
template <int D, bool CHANNEL>
__global__ __launch_bounds__(256) void block_quant_kernel(AppendParams p) {
  constexpr int K = (D + kWave - 1) / kWave;  // element indices per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int w = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int per_side = p.batch * p.geom.kvh * p.nblk;
  if (w >= 2 * per_side) return;
  const int side = w >= per_side ? 1 : 0;
  const int r = w - side * per_side;
  const int jrel = r % p.nblk;
  const int bh = r / p.nblk;
  const int h = bh % p.geom.kvh;
  const int b = bh / p.geom.kvh;
  const int start = p.pos_from_lens ? p.start_pos[b] - 1 : p.start_pos[b];
  const int lo = start - p.rwin;                   // blocks whose first row is in [lo, hi) trigger
  const int hi = start + p.n_new - p.rwin;
  const int j0 = lo <= 0 ? 0 : (lo + kBlockRows - 1) / kBlockRows;
  const int j = j0 + jrel;
  if (start < 0 || kBlockRows * j >= hi) return;
  const int p0 = kBlockRows * j;
  float x[kBlockRows][K];
#pragma unroll
  for (int i = 0; i < kBlockRows; ++i) {
    const int pos = p0 + i;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int d = lane + kWave * k;
      float v = 0.0f;
      if (d < D) {
        if (pos < start) {  // an older row, in its ring slot
          v = bf16_to_f32(p.ring[side][(static_cast<int64_t>(bh) * p.rcap + pos % p.rcap) * D + d]);
        } else {            // this append's row pos - start, entering as bf16
          const int64_t src = (static_cast<int64_t>(bh) * p.n_new + (pos - start)) * D + d;
          const float raw = p.in_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.src[side])[src])
                                      : static_cast<const float*>(p.src[side])[src];
          v = bf16_to_f32(f32_to_bf16_rne(raw));
        }
      }
      x[i][k] = v;
    }
  }
  float s[K];
  if constexpr (CHANNEL) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < kBlockRows; ++i) a = fmaxf(a, fabsf(x[i][k]));
      s[k] = fmaxf(a, 1e-8f) / 127.0f;  // IEEE division (correctly rounded)
    }
  } else {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlockRows; ++i)
#pragma unroll
      for (int k = 0; k < K; ++k) a = fmaxf(a, fabsf(x[i][k]));
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
    const float sh = fmaxf(a, 1e-8f) / 127.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) s[k] = sh;
  }
  int64_t row0 = -1;
#pragma unroll
  for (int i = 0; i < kBlockRows; ++i) {
    const int64_t row = cache_row(p.geom, b, h, p0 + i);
    if (i == 0) row0 = row;
    if (row < 0) continue;  // outside the cache: not written
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int d = lane + kWave * k;
      if (d >= D) continue;
      const float y = x[i][k] / s[k];  // IEEE division, not a reciprocal multiply
      float q = roundf(y);             // half away from zero
      q = fminf(fmaxf(q, -127.0f), 127.0f);
      p.codes[side][row * D + d] = static_cast<uint8_t>(static_cast<int>(q) + 128);
    }
    if (!CHANNEL && lane == 0) p.scales[side][row] = s[0];  // the block's scale on each of its rows
  }
  if (CHANNEL && row0 >= 0) {
    // [row / 16] is the block's slot: contiguous (b, h, j), paged (page, h)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int d = lane + kWave * k;
      if (d < D) p.scales[side][(row0 / kBlockRows) * D + d] = s[k];
    }
  }
}

template <bool CHANNEL>
void launch_block_quant(int head_dim, dim3 grid, hipStream_t st, const AppendParams& p) {
  switch (head_dim) {
    case 32: hipLaunchKernelGGL((block_quant_kernel<32, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((block_quant_kernel<64, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 96: hipLaunchKernelGGL((block_quant_kernel<96, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((block_quant_kernel<128, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 160: hipLaunchKernelGGL((block_quant_kernel<160, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 192: hipLaunchKernelGGL((block_quant_kernel<192, CHANNEL>), grid, dim3(256), 0, st, p); break;
    case 224: hipLaunchKernelGGL((block_quant_kernel<224, CHANNEL>), grid, dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((block_quant_kernel<256, CHANNEL>), grid, dim3(256), 0, st, p); break;
  }
}

// ---------------------------------------------------------------------------
// Dequantization: out = fl32((code - 128) * s) (abaddon kv_cache_quant_cuda.rs
// `int8_dequant_bf16`; abaddon 0.2.0-rc.2 src/kv_cache_quant.rs
// `dequantize`), optionally rounded to bf16.  One thread per 4 elements.
// ---------------------------------------------------------------------------
struct DequantParams {
  const uint8_t* codes;
  const float* scales;
  const uint16_t* ring;      // recent window: bf16 [B, KVH, rcap, D]
  int32_t rwin, rcap;        // window (0: none) and ring slots
  int32_t scale_bf16;        // per-token scales stored as bf16
  int32_t fp8;               // FP8 codes: 1 E4M3, 2 E5M2 (no scales); 0 INT8
  const int32_t* seq_lens;
  void* out;
  CacheGeom geom;
  int32_t batch, head_dim, groups, out_len, out_bf16;
  int32_t channel;  // per-channel block scales: [row / 16][d]
  int64_t quads;  // B * KVH * out_len * D / 4
};

__global__ __launch_bounds__(256) void dequant_kernel(DequantParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= p.quads) return;
  const int D = p.head_dim;
  const int64_t e0 = idx * 4;
  const int d = static_cast<int>(e0 % D);
  const int64_t trow = e0 / D;  // (b*KVH + h)*out_len + t
  const int t = static_cast<int>(trow % p.out_len);
  const int64_t bh = trow / p.out_len;
  const int h = static_cast<int>(bh % p.geom.kvh);
  const int b = static_cast<int>(bh / p.geom.kvh);
  int len = p.seq_lens[b];
  len = len < 0 ? 0 : (len > capacity(p.geom) ? capacity(p.geom) : len);
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // with a recent window the last rwin positions come from the ring (bf16)
  const bool recent = t < len && t >= len - p.rwin;
  const int64_t row = t < len && !recent ? cache_row(p.geom, b, h, t) : -1;
  if (recent) {
    const uint2 r = *reinterpret_cast<const uint2*>(p.ring + (bh * p.rcap + t % p.rcap) * D + d);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  } else if (row >= 0 && p.fp8) {
    // FP8: the page's decoder (llama-gguf kv_quantized.rs `dequantize_fp8_*`)
    const uint32_t c = *reinterpret_cast<const uint32_t*>(p.codes + row * D + d);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = p.fp8 == 2 ? fp8_decode<true>((c >> (8 * e)) & 0xffu) : fp8_decode<false>((c >> (8 * e)) & 0xffu);
  } else if (row >= 0 && p.channel) {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(p.codes + row * D + d);
    const float4 s = *reinterpret_cast<const float4*>(p.scales + (row / kBlockRows) * D + d);
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<float>(static_cast<int>((c >> (8 * e)) & 0xffu) - 128) * sv[e];
  } else if (row >= 0) {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(p.codes + row * D + d);
    const float s = load_scale(p.scales, row * p.groups + (p.groups == 1 ? 0 : d / 32), p.scale_bf16 != 0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<float>(static_cast<int>((c >> (8 * e)) & 0xffu) - 128) * s;
  }
  if (p.out_bf16) {
    ushort4 o;
    o.x = f32_to_bf16_rne(v[0]);
    o.y = f32_to_bf16_rne(v[1]);
    o.z = f32_to_bf16_rne(v[2]);
    o.w = f32_to_bf16_rne(v[3]);
    reinterpret_cast<ushort4*>(p.out)[idx] = o;
  } else {
    reinterpret_cast<float4*>(p.out)[idx] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <bool G32>
void dispatch_epl(int epl, dim3 grid, hipStream_t st, const AppendParams& p) {
  if (epl == 1)
    hipLaunchKernelGGL((append_kernel<1, G32>), grid, dim3(256), 0, st, p);
  else if (epl == 2)
    hipLaunchKernelGGL((append_kernel<2, G32>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((append_kernel<4, G32>), grid, dim3(256), 0, st, p);
}

}  // namespace

kvq_status launch_append(const kvq_cache& c, const void* k_new, const void* v_new, int in_dtype,
                         int n_new, const int32_t* start_pos, hipStream_t stream, bool pos_from_lens,
                         const RecentGeom& rc) {
  AppendParams p;
  p.ring[0] = rc.k;
  p.ring[1] = rc.v;
  p.rwin = rc.window;
  p.rcap = rc.cap;
  p.n_new = n_new;
  p.scale_bf16 = c.scale_mode == KVQ_SCALE_PER_TOKEN_BF16 ? 1 : 0;
  p.fp8 = fp8_kind(c);
  p.src[0] = k_new;
  p.src[1] = v_new;
  p.codes[0] = c.k_codes;
  p.codes[1] = c.v_codes;
  p.scales[0] = c.k_scales;
  p.scales[1] = c.v_scales;
  p.start_pos = start_pos;
  p.geom = geom_of(c);
  p.batch = c.batch;
  p.n = n_new;
  p.head_dim = c.head_dim;
  p.groups = scales_per_row(c);
  p.pos_from_lens = pos_from_lens ? 1 : 0;
  p.in_bf16 = in_dtype == KVQ_DT_BF16 ? 1 : 0;
  p.block = c.scale_mode == KVQ_SCALE_BLOCK_HEAD ? 1 : (c.scale_mode == KVQ_SCALE_BLOCK_CHANNEL ? 2 : 0);
  p.nblk = 0;
  if (p.block) {
    // block scales: first the blocks whose first row leaves the window (at
    // most n_new / 16 + 2 per sequence), then the new rows of the window
    p.nblk = n_new / kBlockRows + 2;
    const int64_t waves = 2ll * c.batch * c.num_kv_heads * p.nblk;
    if (waves > 0x7fffffffLL) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_append_recent: too many blocks");
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    if (p.block == 2) launch_block_quant<true>(c.head_dim, grid, stream, p);
    else launch_block_quant<false>(c.head_dim, grid, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_append_recent: block launch failed: %s", hipGetErrorString(e));
  }
  // one launch per pass: with a recent window, first the ring rows that
  // leave it (at most min(n_new, W) per sequence; the block pass has done
  // that with block scales), then the new rows
  const int passes = rc.window > 0 ? 2 : 1;
  for (int pass = p.block ? 1 : 0; pass < passes; ++pass) {
    p.mode = rc.window == 0 ? kPlain : (pass == 0 ? kEvict : kRows);
    p.n = p.mode == kEvict ? (n_new < rc.window ? n_new : rc.window) : n_new;
    const int64_t rows = static_cast<int64_t>(c.batch) * c.num_kv_heads * p.n;
    if (rows * 2 > 0x7fffffffLL)
      return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_append: too many rows (%lld)", (long long)rows);
    p.rows_per_side = static_cast<int32_t>(rows);
    const int64_t waves = rows * 2;
    dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    if (c.scale_mode == KVQ_SCALE_GROUP32) dispatch_epl<true>(row_epl(c.head_dim), grid, stream, p);
    else dispatch_epl<false>(row_epl(c.head_dim), grid, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_append: launch failed: %s", hipGetErrorString(e));
  }
  return KVQ_OK;
}

kvq_status launch_dequant(const kvq_cache& c, int which, const int32_t* seq_lens, int out_dtype,
                          void* out, int out_len, hipStream_t stream, const RecentGeom& rc) {
  DequantParams p;
  p.ring = which ? rc.v : rc.k;
  p.rwin = rc.window;
  p.rcap = rc.cap;
  p.scale_bf16 = c.scale_mode == KVQ_SCALE_PER_TOKEN_BF16 ? 1 : 0;
  p.fp8 = fp8_kind(c);
  p.codes = which ? c.v_codes : c.k_codes;
  p.scales = which ? c.v_scales : c.k_scales;
  p.seq_lens = seq_lens;
  p.out = out;
  p.geom = geom_of(c);
  p.batch = c.batch;
  p.head_dim = c.head_dim;
  p.groups = c.scale_mode == KVQ_SCALE_BLOCK_HEAD ? 1 : scales_per_row(c);
  p.channel = c.scale_mode == KVQ_SCALE_BLOCK_CHANNEL ? 1 : 0;
  p.out_len = out_len;
  p.out_bf16 = out_dtype == KVQ_DT_BF16 ? 1 : 0;
  p.quads = static_cast<int64_t>(c.batch) * c.num_kv_heads * out_len * c.head_dim / 4;
  if (p.quads == 0) return KVQ_OK;
  const int64_t blocks = (p.quads + 255) / 256;
  if (blocks > 0x7fffffffLL) return fail(KVQ_ERR_OUT_OF_RANGE, "kvq_dequant: output too large");
  hipLaunchKernelGGL(dequant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_dequant: launch failed: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq
