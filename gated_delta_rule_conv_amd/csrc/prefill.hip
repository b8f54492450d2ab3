// Chunked prefill of the gated delta rule (placeholder until the MFMA kernels land).
#include "launch.h"

namespace gdn {

size_t prefill_workspace_bytes(int32_t hv, int32_t d, int32_t chunk, int32_t num_seqs, int32_t total_tokens) {
  (void)d;
  const size_t max_chunks = static_cast<size_t>(total_tokens) / chunk + static_cast<size_t>(num_seqs);
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  return up(max_chunks * 16) + up((static_cast<size_t>(num_seqs) + 1) * 4) + 256 +
         2 * up(max_chunks * hv * chunk * chunk * 4);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace gdn
