// Instantiations of the streaming decode kernel for FP8 codes (llama-gguf
// 0.14.0 src/model/kv_quantized.rs, `KVCacheFormat::Fp8E4M3` / `Fp8E5M2`),
// kept in a translation unit of their own so the library's kernels compile
// in parallel.  The kernel is the one in kvq_decode_stream.hpp; the FP8
// modes decode code pairs to f16 values and carry no scales.
#include "kvq_decode_stream.hpp"

namespace kvq {
namespace {

template <int D, int HPW, int SM>
void launch_fp8(bool paged, bool append, const DecodeParams& p, dim3 grid, hipStream_t st) {
  if (paged) {
    if (append) hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, true, true>), grid, dim3(kStreamThreads), 0, st, p);
    else hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, true, false>), grid, dim3(kStreamThreads), 0, st, p);
  } else {
    if (append) hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, false, true>), grid, dim3(kStreamThreads), 0, st, p);
    else hipLaunchKernelGGL((decode_stream_kernel<D, HPW, SM, false, false>), grid, dim3(kStreamThreads), 0, st, p);
  }
}

template <int D, int HPW>
void launch_fp8_formats(int sm, bool paged, bool append, const DecodeParams& p, dim3 grid, hipStream_t st) {
  if (sm == kSmFp8E5M2) launch_fp8<D, HPW, kSmFp8E5M2>(paged, append, p, grid, st);
  else launch_fp8<D, HPW, kSmFp8E4M3>(paged, append, p, grid, st);
}

template <int D>
void launch_fp8_hpw(int hpw, int sm, bool paged, bool append, const DecodeParams& p, dim3 grid, hipStream_t st) {
  if (hpw == 4) launch_fp8_formats<D, 4>(sm, paged, append, p, grid, st);
  else if (hpw == 2) launch_fp8_formats<D, 2>(sm, paged, append, p, grid, st);
  else launch_fp8_formats<D, 1>(sm, paged, append, p, grid, st);
}

}  // namespace

void launch_stream_fp8(int head_dim, int hpw, int sm, bool paged, bool append, const DecodeParams& p, dim3 grid,
                       hipStream_t st) {
  switch (head_dim) {
    case 32: launch_fp8_hpw<32>(hpw, sm, paged, append, p, grid, st); break;
    case 64: launch_fp8_hpw<64>(hpw, sm, paged, append, p, grid, st); break;
    default: launch_fp8_hpw<128>(hpw, sm, paged, append, p, grid, st); break;
  }
}

}  // namespace kvq
