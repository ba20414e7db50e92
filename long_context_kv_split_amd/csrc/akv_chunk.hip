// Prefill-chunk attention (placeholder until the matrix-core chunk kernel lands).
#include "akv_common.h"
#include "akv_params.h"

namespace akv {
hipError_t launch_chunk(const AttnParams& p, int D, hipStream_t stream) {
  (void)p; (void)D; (void)stream;
  return hipErrorNotSupported;
}
}  // namespace akv
