// Instantiations of the streaming decode kernel (kvq_decode_stream.hpp) for
// INT8 codes with group-32 fp32 scales, in a translation unit of their own so the library's
// kernels compile in parallel.
#include "kvq_decode_stream.hpp"

namespace kvq {

void launch_stream_group32(int head_dim, int hpw, bool paged, bool append, const DecodeParams& p, dim3 grid,
                           hipStream_t st) {
  launch_stream_impl<kSmGroup32>(head_dim, hpw, paged, append, p, grid, st);
}

}  // namespace kvq
