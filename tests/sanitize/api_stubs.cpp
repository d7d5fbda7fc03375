// Host-only stand-ins for the kernel launchers and sizing helpers that
// api.cpp calls (declared in aware_tiling_amd/csrc/launch.h), so that the
// C-ABI validation can be built with the host compiler under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Launchers record the call and touch no
// memory; sizing helpers return simple values of the right kind.  No GPU is
// involved.
#include <hip/hip_runtime.h>

#include <cstring>

#include "launch.h"

int g_launches = 0;
hipError_t g_launch_result = hipSuccess;

extern "C" const char* hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "stubbed launch error";
}

namespace at {

static hipError_t launched() {
  ++g_launches;
  return g_launch_result;
}

bool fused_bf16_supported(int64_t d) { return d == 64 || d == 128 || d == 256; }
bool fused_f32_supported(int64_t d) { return d == 64 || d == 128; }
FusedTileInfo fused_bf16_tile_info(int64_t d, const char* tile) {
  if (!fused_bf16_supported(d)) return FusedTileInfo{0, 0, 0};
  if (tile && std::strcmp(tile, "default") != 0 && std::strcmp(tile, "other") != 0)
    return FusedTileInfo{0, 0, 0};
  return FusedTileInfo{256, 64, 98816};
}
const char* fused_bf16_tile_names(int64_t d) { return fused_bf16_supported(d) ? "default other" : ""; }
FusedTileInfo fused_f32_tile_info(int64_t d) {
  return fused_f32_supported(d) ? FusedTileInfo{128, 32, 1000} : FusedTileInfo{0, 0, 0};
}
hipError_t launch_fwd_fused_bf16(const void*, const void*, const void*, float*, float*, int64_t,
                                 int64_t, int64_t, float, const char*, hipStream_t) {
  return launched();
}
bool fused_budget_supported(int64_t d) { return d == 128 || d == 256; }
int64_t fused_budget_onchip(int64_t d) { return fused_budget_supported(d) ? 54336 : 0; }
hipError_t launch_fwd_budget_bf16(const void*, const void*, const void*, float*, float*, int64_t,
                                  int64_t, int64_t, float, hipStream_t) {
  return launched();
}
hipError_t launch_fwd_fused_f32(const float*, const float*, const float*, float*, float*, int64_t,
                                int64_t, int64_t, float, hipStream_t) {
  return launched();
}
size_t align256_bytes(size_t b) { return (b + 255) / 256 * 256; }
bool splitk_supported(int64_t d) { return d == 64 || d == 128; }
int64_t splitk_auto_splits(int64_t, int64_t, int64_t nk, int64_t) { return nk > 1024 ? 4 : 1; }
int64_t splitk_key_chunk(int64_t nk, int64_t splits) {
  const int64_t per = (nk + splits - 1) / splits;
  return (per + 63) / 64 * 64;
}
int64_t splitk_effective_splits(int64_t nk, int64_t splits) {
  const int64_t kc = splitk_key_chunk(nk, splits);
  return (nk + kc - 1) / kc;
}
size_t splitk_workspace_bytes(int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t splits) {
  if (splitk_effective_splits(nk, splits) <= 1) return 0;
  return align256_bytes((size_t)(splits * bh * nq * d) * 4) + align256_bytes((size_t)(splits * bh * nq) * 4);
}
hipError_t launch_fwd_splitk_bf16(const void*, const void*, const void*, float*, float*, int64_t,
                                  int64_t, int64_t, int64_t, float, int64_t, void*, hipStream_t) {
  return launched();
}
hipError_t launch_fwd_splitk_noalloc_bf16(const void*, const void*, const void*, float*, float*,
                                          int64_t, int64_t, int64_t, int64_t, float, int64_t,
                                          hipStream_t) {
  return launched();
}
size_t sparse_workspace_bytes(int64_t n, int64_t mask_heads) {
  const int64_t nqb = (n + kSparseBlock - 1) / kSparseBlock, cap = (n + 63) / 64;
  return align256_bytes((size_t)(mask_heads * nqb) * 4) + align256_bytes((size_t)(mask_heads * nqb * cap) * 4);
}
hipError_t launch_fwd_sparse_bf16(const void*, const void*, const void*, float*, float*, int64_t,
                                  int64_t, int64_t, float, const uint8_t*, int64_t, void*,
                                  hipStream_t) {
  return launched();
}
bool smallcache_supported(int64_t d) { return d == 128 || d == 256; }
int64_t smallcache_tile_for_budget(int64_t d, int64_t m) {
  if (!smallcache_supported(d)) return 0;
  return m >= 40960 ? 128 : m >= 12288 ? 64 : 0;
}
int64_t smallcache_onchip_elems(int64_t b) { return b == 128 ? 40960 : b == 64 ? 12288 : 0; }
size_t smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b) {
  const int64_t np = (n + b - 1) / b * b;
  return align256_bytes((size_t)(bh * np * np) * 2) + 2 * align256_bytes((size_t)(bh * (np / b) * n) * 4);
}
hipError_t launch_fwd_smallcache_bf16(const void*, const void*, const void*, float*, float*,
                                      int64_t, int64_t, int64_t, float, int64_t, void*,
                                      hipStream_t) {
  return launched();
}
bool bwd_supported(int64_t d) { return d == 64 || d == 128; }
int64_t bwd_onchip_elems(int64_t d) { return bwd_supported(d) ? 1 : 0; }
BwdTileInfo bwd_tile_info(int64_t d, const char* tile) {
  if (!bwd_supported(d)) return BwdTileInfo{0, 0, 0, 0};
  if (tile == nullptr || std::strcmp(tile, "k256q256c64") == 0) return BwdTileInfo{256, 256, 64, 1};
  return BwdTileInfo{0, 0, 0, 0};
}
const char* bwd_tile_names(int64_t d) { return bwd_supported(d) ? "k256q256c64" : ""; }
size_t bwd_workspace_bytes(int64_t bh, int64_t n, int64_t) { return 2 * align256_bytes((size_t)bh * n * 4); }
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const float*, const void*,
                           const float*, float*, float*, float*, int64_t, int64_t, int64_t, float,
                           void*, const char*, hipStream_t) {
  return launched();
}
bool bwd_smallcache_supported(int64_t d) { return d == 128 || d == 256; }
int64_t bwd_smallcache_onchip_elems(int64_t b, int64_t stages) { return 2 * b * b + 4 * b * 16 * stages; }
SmallBwdTile bwd_smallcache_tile(int64_t d, int64_t m) {
  if (!bwd_smallcache_supported(d) || m <= 0 || m >= d * d) return SmallBwdTile{0, 0};
  if (m >= 49152) return SmallBwdTile{128, 2};
  if (m >= 12288) return SmallBwdTile{64, 1};
  return SmallBwdTile{0, 0};
}
size_t bwd_smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b) {
  const int64_t np = (n + b - 1) / b * b;
  return align256_bytes((size_t)bh * n * 4) + 2 * align256_bytes((size_t)(bh * np * np) * 2);
}
hipError_t launch_bwd_smallcache_bf16(const void*, const void*, const void*, const float*,
                                      const void*, const float*, float*, float*, float*, int64_t,
                                      int64_t, int64_t, float, SmallBwdTile, void*, hipStream_t) {
  return launched();
}
hipError_t launch_calib_mfma_loop(float*, int64_t, int, float, hipStream_t) { return launched(); }
hipError_t launch_calib_stream_read(const void*, int64_t, uint32_t*, int64_t, hipStream_t) { return launched(); }

}  // namespace at
