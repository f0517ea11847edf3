// Chunked-prefill attention over a paged KV cache (matrix-core kernel).
#include "common.h"
#include "device_utils.h"

namespace pkv {

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  (void)p;
  (void)head_dim;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pkv
