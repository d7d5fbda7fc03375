// Square-tile (small-cache) forward: not built yet; the C ABI reports
// ATTN_ERR_UNSUPPORTED for it.
#include "launch.h"

namespace at {
bool smallcache_supported(int64_t) { return false; }
int64_t smallcache_tile_for_budget(int64_t, int64_t) { return 0; }
int64_t smallcache_onchip_elems(int64_t) { return 0; }
size_t smallcache_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
hipError_t launch_fwd_smallcache_bf16(const void*, const void*, const void*, float*, float*,
                                      int64_t, int64_t, int64_t, float, int64_t, void*,
                                      hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace at
