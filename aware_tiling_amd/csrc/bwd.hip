// Backward: not built yet; the C ABI reports ATTN_ERR_UNSUPPORTED for it.
#include "launch.h"

namespace at {
bool bwd_supported(int64_t) { return false; }
size_t bwd_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const float*, const void*,
                           const float*, float*, float*, float*, int64_t, int64_t, int64_t,
                           float, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace at
