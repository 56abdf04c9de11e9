// Row quantizer shared by the append kernel and the fused append+decode
// kernel: one wave64 holds one token row of D values, EPL per lane.
//
// Steps of abaddon 0.2.0-rc.1 src/kv_cache_quant_cuda.rs,
// `CudaQuantizedKvCache::quantize_tensor`, in IEEE fp32:
//   m = max(max|x|, 1e-8); s = m / 127; q = round-half-away(x / s); code = q + 128
// with the maximum taken over the row or over each 32-element group
// (combs-models 0.2.2 src/kv.rs, `kv_quantize`).  Divisions are correctly
// rounded (the build keeps -fhip-fp32-correctly-rounded-divide-sqrt) and the
// maximum is exact, so the reduction order cannot change a code.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

// Smallest power of two EPL with D / EPL <= 64.
constexpr int row_epl(int head_dim) { return head_dim <= 64 ? 1 : (head_dim <= 128 ? 2 : 4); }

// Loads this lane's EPL consecutive values of a row as fp32 (bf16 widened
// exactly).  `bf16` selects the input format at run time.
template <int EPL>
__device__ __forceinline__ void load_row_values(const void* row, int lane, bool active, bool bf16,
                                                float (&x)[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = 0.0f;
  if (!active) return;
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + lane * EPL;
    if constexpr (EPL == 1) {
      x[0] = bf16_to_f32(p[0]);
    } else if constexpr (EPL == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
      x[0] = __uint_as_float(v << 16);
      x[1] = __uint_as_float(v & 0xffff0000u);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      x[0] = __uint_as_float(v.x << 16);
      x[1] = __uint_as_float(v.x & 0xffff0000u);
      x[2] = __uint_as_float(v.y << 16);
      x[3] = __uint_as_float(v.y & 0xffff0000u);
    }
  } else {
    const float* p = static_cast<const float*>(row) + lane * EPL;
    if constexpr (EPL == 1) {
      x[0] = p[0];
    } else if constexpr (EPL == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      x[0] = v.x;
      x[1] = v.y;
    } else {
      const float4 v = *reinterpret_cast<const float4*>(p);
      x[0] = v.x;
      x[1] = v.y;
      x[2] = v.z;
      x[3] = v.w;
    }
  }
}

// Codes of this lane's EPL values, packed little-endian, and the scale of
// the row (per-token) or of this lane's 32-element group (GROUP32).  Every
// lane of the wave must call it; lanes without values pass zeros.
template <int EPL, bool GROUP32>
__device__ __forceinline__ uint32_t quantize_lane(const float (&x)[EPL], float& scale) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
  constexpr int kGroupLanes = 32 / EPL;
  constexpr int kSpan = GROUP32 ? kGroupLanes : kWave;
#pragma unroll
  for (int off = kSpan / 2; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
  const float m = fmaxf(a, 1e-8f);
  const float s = m / 127.0f;  // IEEE division (correctly rounded)
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float y = x[e] / s;  // IEEE division, not a reciprocal multiply
    float q = roundf(y);       // half away from zero
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    packed |= static_cast<uint32_t>(static_cast<int>(q) + 128) << (8 * e);
  }
  scale = s;
  return packed;
}

// Stores this lane's EPL codes of a row that starts at `codes`.
template <int EPL>
__device__ __forceinline__ void store_lane_codes(uint8_t* codes, int lane, uint32_t packed) {
  uint8_t* out = codes + lane * EPL;
  if constexpr (EPL == 1) {
    *out = static_cast<uint8_t>(packed);
  } else if constexpr (EPL == 2) {
    *reinterpret_cast<uint16_t*>(out) = static_cast<uint16_t>(packed);
  } else {
    *reinterpret_cast<uint32_t*>(out) = packed;
  }
}

}  // namespace kvq
