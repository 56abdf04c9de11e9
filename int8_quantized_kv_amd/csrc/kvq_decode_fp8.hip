// Instantiations of the streaming decode kernel for FP8 codes (llama-gguf
// 0.14.0 src/model/kv_quantized.rs, `KVCacheFormat::Fp8E4M3` / `Fp8E5M2`),
// kept in a translation unit of their own so the library's kernels compile
// in parallel.  The kernel is the one in kvq_decode_stream.hpp; the FP8
// modes decode code pairs to f16 values and carry no scales.
#include "kvq_decode_stream.hpp"

namespace kvq {

void launch_stream_fp8(int head_dim, int hpw, int sm, bool paged, bool append, const DecodeParams& p, dim3 grid,
                       hipStream_t st) {
  if (sm == kSmFp8E5M2) launch_stream_impl<kSmFp8E5M2>(head_dim, hpw, paged, append, p, grid, st);
  else launch_stream_impl<kSmFp8E4M3>(head_dim, hpw, paged, append, p, grid, st);
}

}  // namespace kvq
