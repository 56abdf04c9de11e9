// Chunked-prefill attention on the INT8 cache (bf16 MFMA).  Placeholder until
// the MFMA kernel lands: reports the call as unsupported.
#include "kvq_internal.hpp"

namespace kvq {

bool chunk_supported(int) { return false; }

size_t chunk_workspace(const kvq_cache&, int, int) { return 0; }

kvq_status launch_chunk(const kvq_cache&, const uint16_t*, int, const int32_t*, int, float, uint16_t*, void*,
                        int, hipStream_t) {
  return fail(KVQ_ERR_UNSUPPORTED, "kvq_attention_chunk: not available");
}

}  // namespace kvq
