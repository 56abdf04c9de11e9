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

// Codes of this lane's EPL values under a given scale s, packed little-endian.
template <int EPL>
__device__ __forceinline__ uint32_t codes_with_scale(const float (&x)[EPL], float s) {
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float y = x[e] / s;  // IEEE division, not a reciprocal multiply
    float q = roundf(y);       // half away from zero
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    packed |= static_cast<uint32_t>(static_cast<int>(q) + 128) << (8 * e);
  }
  return packed;
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
  scale = s;
  return codes_with_scale(x, s);
}

// Stores this lane's EPL codes of a row that starts at `codes`.
// The same values in two steps: the raw bytes of this lane's EPL elements
// (fp32 or bf16, up to 16 bytes), and their fp32 values.  Splitting them
// lets a load go out early while its conversion waits for the use, so the
// load is not waited for on the spot.
template <int EPL>
__device__ __forceinline__ uint4 load_row_raw(const void* row, int lane, bool active, bool bf16) {
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  if (!active) return r;
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + lane * EPL;
    if constexpr (EPL == 1) r.x = p[0];
    else if constexpr (EPL == 2) r.x = *reinterpret_cast<const uint32_t*>(p);
    else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      r.x = v.x;
      r.y = v.y;
    }
  } else {
    const float* p = static_cast<const float*>(row) + lane * EPL;
    if constexpr (EPL == 1) r.x = __float_as_uint(p[0]);
    else if constexpr (EPL == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      r.x = v.x;
      r.y = v.y;
    } else {
      r = *reinterpret_cast<const uint4*>(p);
    }
  }
  return r;
}

template <int EPL>
__device__ __forceinline__ void row_raw_values(uint4 r, bool bf16, float (&x)[EPL]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if (bf16) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float(w[e]);
  }
}

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

namespace kvq {

// ---------------------------------------------------------------------------
// FP8 codes (llama-gguf 0.14.0 src/model/kv_quantized.rs, `quantize_fp8_e4m3`
// / `quantize_fp8_e5m2`, `dequantize_fp8_*`): one byte per element, no scale.
// E4M3: 3 mantissa bits, bias 7; E5M2: 2 mantissa bits, bias 15.
// ---------------------------------------------------------------------------

// The page's encoder: NaN -> 0xFF, +/-inf -> the infinity code, +/-0 -> 0;
// otherwise the fp32 exponent is rebased, an exponent above the largest
// field gives the overflow code (E4M3 +/-448, E5M2 +/-inf), a normal result
// keeps the top mantissa bits, a subnormal one the top bits of the full
// significand, and anything smaller a signed zero: the value is cut toward
// zero, never rounded.
template <bool E5M2>
__device__ __forceinline__ uint32_t fp8_encode(float x) {
  constexpr int M = E5M2 ? 2 : 3;
  constexpr int kBias = E5M2 ? 15 : 7;
  constexpr int kEmax = E5M2 ? 31 : 15;
  constexpr uint32_t kMask = (1u << M) - 1;
  const uint32_t u = __float_as_uint(x);
  const uint32_t s7 = (u >> 24) & 0x80u;
  const int raw = static_cast<int>((u >> 23) & 0xFFu);
  const uint32_t sig = (u & 0x7FFFFFu) | (raw != 0 ? 0x800000u : 0u);
  const int E = raw - 127 + kBias;
  if (x != x) return 0xFFu;
  if (raw == 0xFF) return s7 | (E5M2 ? 0x7Cu : 0x7Fu);
  if ((u & 0x7FFFFFFFu) == 0) return 0u;
  if (E > kEmax) return s7 | (E5M2 ? 0x7Cu : 0x7Eu);
  if (E >= 1) return s7 | (static_cast<uint32_t>(E) << M) | ((sig >> (23 - M)) & kMask);
  if (E > -M) return s7 | ((sig >> (24 - M - E)) & (kMask >> (-E)));
  return s7;
}

// The page's decoder, exact in fp32: a zero magnitude is +0 (either sign),
// E4M3 S.1111.111 is NaN, E5M2 S.11111.00 is +/-inf and above it NaN; a
// nonzero exponent field F gives 2^(F - bias) (1 + f / 2^M), F = 0 the
// subnormal f 2^(1 - bias - M).
template <bool E5M2>
__device__ __forceinline__ float fp8_decode(uint32_t c) {
  constexpr int M = E5M2 ? 2 : 3;
  constexpr int kBias = E5M2 ? 15 : 7;
  const uint32_t low = c & 0x7Fu;
  const uint32_t sign = (c & 0x80u) << 24;
  if (low == 0) return 0.0f;
  if (!E5M2 && low == 0x7Fu) return __uint_as_float(0x7FC00000u);
  if (E5M2 && low == 0x7Cu) return __uint_as_float(sign | 0x7F800000u);
  if (E5M2 && low > 0x7Cu) return __uint_as_float(0x7FC00000u);
  const uint32_t F = low >> M, f = low & ((1u << M) - 1);
  if (F > 0) return __uint_as_float(sign | ((F + 127u - kBias) << 23) | (f << (23 - M)));
  return __uint_as_float(sign | __float_as_uint(static_cast<float>(f) * (E5M2 ? 0x1p-16f : 0x1p-9f)));
}

// FP8 codes of this lane's EPL values, packed little-endian.
template <int EPL, bool E5M2>
__device__ __forceinline__ uint32_t fp8_encode_lane(const float (&x)[EPL]) {
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) packed |= fp8_encode<E5M2>(x[e]) << (8 * e);
  return packed;
}

// FP8 code pairs as f16 pairs (every E4M3 and E5M2 value, infinities and
// NaN included, is an f16 value).  E5M2 is the upper byte of an f16; E4M3
// goes through gfx950's conversion (scale 1), which decodes every byte as
// the OCP format does.  fp8_pair_k: bytes (0, 1) or (2, 3) of w.
template <bool E5M2, bool HIGH>
__device__ __forceinline__ uint32_t fp8_pair_k(uint32_t w) {
  if constexpr (E5M2) {
    return __builtin_amdgcn_perm(0u, w, HIGH ? 0x030C020Cu : 0x010C000Cu);
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
  }
}

// Byte e of a and byte e of b (two tokens' codes of one dim) as an f16 pair.
template <bool E5M2>
__device__ __forceinline__ uint32_t fp8_pair_v(uint32_t a, uint32_t b, int e) {
  if constexpr (E5M2) {
    return __builtin_amdgcn_perm(b, a, 0x040C000Cu + 0x01000100u * e);
  } else {
    return __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(b, a, 0x0C0C0400u + 0x0101u * e),
                                                           1.0f, false));
  }
}

}  // namespace kvq
