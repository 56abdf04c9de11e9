// Read-bandwidth probe: a kernel that only streams a device buffer through
// 16-byte vector loads.  It is the measured ceiling that the decode kernels'
// achieved bandwidth is compared with (HBM bytes per second that a plain read
// stream reaches on this chip, for the same byte count per launch).
#include "kvq_internal.hpp"

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace kvq {
namespace {

constexpr uint32_t kNever = 0x9E3779B9u;  // xor of everything read; written out only if equal

// Each wave keeps between U and 2U 1-KB loads in flight (two register sets:
// one is consumed while the other's loads are outstanding).  INTERLEAVE: the
// waves of a workgroup take turns over 64*U-word steps of the workgroup's
// contiguous range (as the decode kernel's waves take turns over blocks);
// otherwise each wave reads a contiguous range of its own.  NT: non-temporal
// loads (as the decode kernels read K and V codes).
template <int U, bool INTERLEAVE, bool NT>
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                           uint32_t* sink) {
  const int waves = blockDim.x / kWave;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  constexpr int64_t kStep = static_cast<int64_t>(kWave) * U;  // words per register set
  int64_t beg, end, stride;
  if constexpr (INTERLEAVE) {
    const int64_t per = ((n16 + gridDim.x - 1) / gridDim.x + kStep - 1) / kStep * kStep;
    const int64_t wg0 = static_cast<int64_t>(blockIdx.x) * per;
    beg = wg0 + wave * kStep;
    end = min(wg0 + per, n16);
    stride = kStep * waves;
  } else {
    const int64_t nw = static_cast<int64_t>(gridDim.x) * waves;
    const int64_t per = ((n16 + nw - 1) / nw + kStep - 1) / kStep * kStep;
    beg = (static_cast<int64_t>(blockIdx.x) * waves + wave) * per;
    end = min(beg + per, n16);
    stride = kStep;
  }
  uint32_t acc = 0;
  uint4 a[U], b[U];
  auto load = [&](uint4 (&r)[U], int64_t i0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * kWave + lane;
      if constexpr (NT) {
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        const v4u v = i < end ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src + i)) : v4u{0u, 0u, 0u, 0u};
        r[u] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        r[u] = i < end ? src[i] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto eat = [&](const uint4 (&r)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  };
  if (beg < end) {
    load(a, beg);
    for (int64_t i = beg; i < end; i += 2 * stride) {
      load(b, i + stride);
      eat(a);
      load(a, i + 2 * stride);
      eat(b);
    }
  }
  if (acc == kNever) sink[0] = acc;
}

template <bool IL, bool NT>
void launch_stream(int depth, const uint4* src, int64_t n16, uint32_t* sink, dim3 grid, dim3 block, hipStream_t st) {
  switch (depth) {
    case 1: hipLaunchKernelGGL((stream_read_kernel<1, IL, NT>), grid, block, 0, st, src, n16, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<2, IL, NT>), grid, block, 0, st, src, n16, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<4, IL, NT>), grid, block, 0, st, src, n16, sink); break;
    default: hipLaunchKernelGGL((stream_read_kernel<8, IL, NT>), grid, block, 0, st, src, n16, sink); break;
  }
}

}  // namespace
}  // namespace kvq

using namespace kvq;

KVQ_API kvq_status kvq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                                   int32_t waves_per_wg, int32_t depth, int32_t interleave, void* stream) {
  const char* who = "kvq_stream_read";
  if (!src || !sink) return fail(KVQ_ERR_INVALID_ARG, "%s: src and sink must be non-NULL", who);
  if (bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return fail(KVQ_ERR_INVALID_ARG, "%s: bytes must be a positive multiple of 16 and src 16-byte aligned", who);
  if (workgroups < 1 || workgroups > 1 << 20)
    return fail(KVQ_ERR_INVALID_ARG, "%s: workgroups must be in [1, 2^20] (got %d)", who, workgroups);
  if (waves_per_wg < 1 || waves_per_wg > 16)
    return fail(KVQ_ERR_INVALID_ARG, "%s: waves_per_wg must be in [1, 16] (got %d)", who, waves_per_wg);
  if (depth != 1 && depth != 2 && depth != 4 && depth != 8)
    return fail(KVQ_ERR_INVALID_ARG, "%s: depth must be 1, 2, 4 or 8 (got %d)", who, depth);
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const auto* s = static_cast<const uint4*>(src);
  const dim3 grid(workgroups), block(waves_per_wg * kWave);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (interleave & ~3)
    return fail(KVQ_ERR_INVALID_ARG, "%s: interleave takes bits 0 and 1 only (got %d)", who, interleave);
  const bool il = (interleave & 1) != 0, nt = (interleave & 2) != 0;
  if (il && nt) launch_stream<true, true>(depth, s, n16, sink, grid, block, st);
  else if (il) launch_stream<true, false>(depth, s, n16, sink, grid, block, st);
  else if (nt) launch_stream<false, true>(depth, s, n16, sink, grid, block, st);
  else launch_stream<false, false>(depth, s, n16, sink, grid, block, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return KVQ_OK;
}
