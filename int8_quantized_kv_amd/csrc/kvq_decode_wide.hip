// Instantiations of the generic decode kernel (kvq_decode_generic.hpp) at the
// head dims whose 16-byte lane count is not a power of two (96, 160, 192,
// 224), in a translation unit of their own so the library's kernels compile
// in parallel.
#include "kvq_decode_generic.hpp"

namespace kvq {

void launch_generic_wide(int head_dim, int hpw, int sm, bool paged, const DecodeParams& p, dim3 grid,
                         hipStream_t st) {
  switch (head_dim) {
    case 96: launch_generic_all<96>(hpw, sm, paged, p, grid, st); break;
    case 160: launch_generic_all<160>(hpw, sm, paged, p, grid, st); break;
    case 192: launch_generic_all<192>(hpw, sm, paged, p, grid, st); break;
    default: launch_generic_all<224>(hpw, sm, paged, p, grid, st); break;
  }
}

}  // namespace kvq
