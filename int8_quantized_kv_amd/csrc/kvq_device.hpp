// Device helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kWave = 64;
constexpr int kPageSize = 16;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an fp32 word; narrowing rounds to
// nearest with ties to even (abaddon kv_cache_quant_cuda.rs kernel helpers
// define the same format).  NaN stays a quiet NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

// Per-row scales are fp32, or bf16 in the same array's memory (bf16-stored
// per-token scales: abaddon kv_cache_quant_cuda.rs `CudaQuantizedKvCache`
// keeps its scales as BF16).
__device__ __forceinline__ float load_scale(const float* scales, int64_t idx, bool bf16) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(scales)[idx]) : scales[idx];
}

// The same, split in two so that a pipelined load is not waited for at once:
// scale_word loads the 32-bit word holding the scale (for bf16, the aligned
// word containing it; the array must be 4-byte aligned, so the word never
// crosses a page), scale_sel records which half, and scale_value decodes the
// word where the scale is used.
__device__ __forceinline__ uint32_t scale_word(const float* scales, int64_t idx, bool bf16) {
  return reinterpret_cast<const uint32_t*>(scales)[idx >> (bf16 ? 1 : 0)];
}
__device__ __forceinline__ uint32_t scale_sel(int64_t idx, bool bf16) {
  return bf16 ? static_cast<uint32_t>(idx & 1) : 2u;
}
__device__ __forceinline__ float scale_value(uint32_t w, uint32_t sel) {
  return __uint_as_float(sel == 2u ? w : (sel ? (w & 0xffff0000u) : (w << 16)));
}

// Stores a scale and returns the value a reader will get back.
__device__ __forceinline__ float store_scale(float* scales, int64_t idx, float s, bool bf16) {
  if (!bf16) {
    scales[idx] = s;
    return s;
  }
  const uint16_t h = f32_to_bf16_rne(s);
  reinterpret_cast<uint16_t*>(scales)[idx] = h;
  return bf16_to_f32(h);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.  DPP row controls (GFX9 encoding).
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141, // lane i <- lane 7-i inside each 8-lane half row
  kDppRowMirror = 0x140,     // lane i <- lane 15-i inside each 16-lane row
  kDppRowRor8 = 0x128,       // rotate right by 8 inside each 16-lane row
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N in {1,2,4,8,16}); every
// lane of the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

// ---------------------------------------------------------------------------
// Cache addressing.  Returns the row index (token row of one KV head) whose
// codes start at row*D and scales at row*G, or -1 when the position is outside
// the cache (out-of-range page id, unmapped block, position past capacity).
// ---------------------------------------------------------------------------
struct CacheGeom {
  int32_t kvh;          // KV heads
  int32_t max_len;      // contiguous capacity per sequence
  int32_t paged;        // 0/1
  int32_t num_pages;
  int32_t max_blocks;   // block-table row length
  const int32_t* block_table;
};

__device__ __forceinline__ int64_t cache_row(const CacheGeom& g, int b, int h, int pos) {
  if (!g.paged) {
    if (pos < 0 || pos >= g.max_len) return -1;
    return (static_cast<int64_t>(b) * g.kvh + h) * g.max_len + pos;
  }
  if (pos < 0 || pos >= g.max_blocks * kPageSize) return -1;
  int phys = g.block_table[static_cast<int64_t>(b) * g.max_blocks + (pos >> 4)];
  if (phys < 0 || phys >= g.num_pages) return -1;
  return (static_cast<int64_t>(phys) * g.kvh + h) * kPageSize + (pos & (kPageSize - 1));
}

__device__ __forceinline__ int capacity(const CacheGeom& g) {
  return g.paged ? g.max_blocks * kPageSize : g.max_len;
}

}  // namespace kvq
