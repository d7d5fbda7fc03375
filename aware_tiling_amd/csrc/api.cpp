// C-ABI entry points (include/aware_tiling.h): argument validation, kernel
// selection and the HIP error translation.  No entry point allocates device
// memory; every check happens before the first HIP call.
#include "aware_tiling.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "launch.h"

namespace {

static_assert(ATTN_SPLITK_NOALLOC_SCRATCH_BYTES == at::kSplitkScratchBytes,
              "header and library agree on the no-allocation scratch size");

thread_local char g_last_hip_error[256] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

attn_status launch_status(hipError_t e) {
  if (e == hipSuccess) {
    g_last_hip_error[0] = '\0';
    return ATTN_OK;
  }
  std::strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return ATTN_ERR_LAUNCH;
}

// Shapes: bh, n >= 0; per-head element count and the grid must fit the
// kernels' 32-bit in-head indexing.  bh * n <= 2^29 rows keeps every
// one-workgroup-per-block grid inside 32 bits; at d >= 64 that many rows of
// Q, K, V and O would not fit in HBM anyway.
// Every factor is bounded before any product is formed, so no check can
// overflow whatever the caller passes.
bool shape_ok(int64_t bh, int64_t n, int64_t d) {
  if (bh < 0 || n < 0 || d <= 0) return false;
  if (n > (int64_t(1) << 24) || d > (int64_t(1) << 16) || bh > (int64_t(1) << 20)) return false;
  if (n * d >= (int64_t(1) << 31)) return false;
  if (bh * n > (int64_t(1) << 29)) return false;
  return true;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
    default: break;
  }
  return "ATTN_STATUS_UNKNOWN";
}

const char* attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_version(void) { return "0.1.0"; }

int64_t attn_fwd_onchip_elems(int64_t d, attn_dtype dtype) {
  if (dtype == ATTN_BF16) return at::fused_bf16_tile_info(d).onchip;
  if (dtype == ATTN_F32) return at::fused_f32_tile_info(d).onchip;
  return 0;
}

int64_t attn_fwd_query_block(int64_t d, attn_dtype dtype) {
  if (dtype == ATTN_BF16) return at::fused_bf16_tile_info(d).block_rows;
  if (dtype == ATTN_F32) return at::fused_f32_tile_info(d).block_rows;
  return 0;
}

attn_status attn_fwd(const void* Q, const void* K, const void* V, float* O, float* lse,
                     int64_t bh, int64_t n, int64_t d, float scale, attn_dtype dtype,
                     void* stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_BF16 ? !at::fused_bf16_supported(d) : !at::fused_f32_supported(d))
    return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16)
    return launch_status(at::launch_fwd_fused_bf16(Q, K, V, O, lse, bh, n, d, scale, nullptr, s));
  return launch_status(at::launch_fwd_fused_f32(static_cast<const float*>(Q),
                                                static_cast<const float*>(K),
                                                static_cast<const float*>(V), O, lse, bh, n, d,
                                                scale, s));
}

const char* attn_fwd_tiles(int64_t d) { return at::fused_bf16_tile_names(d); }

attn_status attn_fwd_tile_info(const char* tile, int64_t d, int64_t* block_rows,
                               int64_t* key_tile, int64_t* onchip_elems) {
  if (!tile) return ATTN_ERR_INVALID_ARG;
  const at::FusedTileInfo t = at::fused_bf16_tile_info(d, tile);
  if (t.block_rows == 0) return ATTN_ERR_UNSUPPORTED;
  if (block_rows) *block_rows = t.block_rows;
  if (key_tile) *key_tile = t.key_tile;
  if (onchip_elems) *onchip_elems = t.onchip;
  return ATTN_OK;
}

attn_status attn_fwd_tile(const char* tile, const void* Q, const void* K, const void* V,
                          float* O, float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                          attn_dtype dtype, void* stream) {
  if (!tile) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (at::fused_bf16_tile_info(d, tile).block_rows == 0) return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  return launch_status(at::launch_fwd_fused_bf16(Q, K, V, O, lse, bh, n, d, scale, tile,
                                                 static_cast<hipStream_t>(stream)));
}

int64_t attn_fwd_budget_onchip_elems(int64_t d) { return at::fused_budget_onchip(d); }

attn_status attn_fwd_budget(const void* Q, const void* K, const void* V, float* O, float* lse,
                            int64_t bh, int64_t n, int64_t d, float scale, attn_dtype dtype,
                            int64_t m_elems, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale) || m_elems <= 0) return ATTN_ERR_INVALID_ARG;
  if (!at::fused_budget_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (at::fused_budget_onchip(d) > m_elems) return ATTN_ERR_UNSUPPORTED;
  if (bh * ((n + 31) / 32) > INT32_MAX) return ATTN_ERR_INVALID_ARG;  // one workgroup per 32 rows
  if (bh * n == 0) return ATTN_OK;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  return launch_status(at::launch_fwd_budget_bf16(Q, K, V, O, lse, bh, n, d, scale,
                                                  static_cast<hipStream_t>(stream)));
}

namespace {

// Effective split count of attn_fwd_splitk, or 0 if the request is invalid.
int64_t splitk_count(int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t splits) {
  if (splits < 0 || splits > 256 || nk <= 0) return 0;
  const int64_t req = splits == 0 ? at::splitk_auto_splits(bh, nq, nk, d) : splits;
  return req;
}

}  // namespace

int64_t attn_fwd_splitk_splits(int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t splits) {
  if (!shape_ok(bh, nq, d) || !shape_ok(bh, nk, d) || !at::splitk_supported(d)) return 0;
  const int64_t req = splitk_count(bh, nq, nk, d, splits);
  return req ? at::splitk_effective_splits(nk, req) : 0;
}

size_t attn_fwd_splitk_workspace_size(int64_t bh, int64_t nq, int64_t nk, int64_t d,
                                      int64_t splits) {
  if (!shape_ok(bh, nq, d) || !shape_ok(bh, nk, d) || !at::splitk_supported(d)) return 0;
  const int64_t req = splitk_count(bh, nq, nk, d, splits);
  return req ? at::splitk_workspace_bytes(bh, nq, nk, d, req) : 0;
}

attn_status attn_fwd_splitk(const void* Q, const void* K, const void* V, float* O, float* lse,
                            int64_t bh, int64_t nq, int64_t nk, int64_t d, float scale,
                            attn_dtype dtype, int64_t splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, nq, d) || !shape_ok(bh, nk, d) || !scale_ok(scale))
    return ATTN_ERR_INVALID_ARG;
  if (!at::splitk_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (splits < 0 || splits > 256) return ATTN_ERR_INVALID_ARG;
  if (bh * nq == 0) return ATTN_OK;
  if (nk == 0) return ATTN_ERR_INVALID_ARG;  // softmax over no keys is undefined
  const int64_t req = splitk_count(bh, nq, nk, d, splits);
  const int64_t eff = at::splitk_effective_splits(nk, req);
  if (eff * bh * ((nq + 127) / 128) >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  const size_t need = at::splitk_workspace_bytes(bh, nq, nk, d, req);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned256(workspace)))
    return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_fwd_splitk_bf16(Q, K, V, O, lse, bh, nq, nk, d, scale, req,
                                                  workspace, static_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_splitk_noalloc(const void* Q, const void* K, const void* V, float* O,
                                    float* lse, int64_t bh, int64_t nq, int64_t nk, int64_t d,
                                    float scale, attn_dtype dtype, int64_t splits, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, nq, d) || !shape_ok(bh, nk, d) || !scale_ok(scale))
    return ATTN_ERR_INVALID_ARG;
  if (!at::splitk_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (splits < 0 || splits > 256) return ATTN_ERR_INVALID_ARG;
  if (bh * nq == 0) return ATTN_OK;
  if (nk == 0) return ATTN_ERR_INVALID_ARG;
  const int64_t req = splitk_count(bh, nq, nk, d, splits);
  const int64_t eff = at::splitk_effective_splits(nk, req);
  if (eff * bh * ((nq + 127) / 128) >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (at::splitk_workspace_bytes(bh, nq, nk, d, req) > at::kSplitkScratchBytes)
    return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_fwd_splitk_noalloc_bf16(Q, K, V, O, lse, bh, nq, nk, d, scale,
                                                          req, static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_blocksparse_workspace_size(int64_t bh, int64_t n, int64_t mask_heads) {
  if (!shape_ok(bh, n, 64) || !(mask_heads == 1 || mask_heads == bh)) return 0;
  return at::sparse_workspace_bytes(n, mask_heads);
}

attn_status attn_fwd_blocksparse(const void* Q, const void* K, const void* V, float* O,
                                 float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                 attn_dtype dtype, const uint8_t* block_mask,
                                 int64_t mask_heads, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  if (!(mask_heads == 1 || mask_heads == bh) || !block_mask) return ATTN_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  const size_t need = at::sparse_workspace_bytes(n, mask_heads);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_fwd_sparse_bf16(Q, K, V, O, lse, bh, n, d, scale, block_mask,
                                                  mask_heads, workspace,
                                                  static_cast<hipStream_t>(stream)));
}

int64_t attn_smallcache_tile(int64_t d, int64_t m_elems) {
  if (!at::smallcache_supported(d) || m_elems >= d * d) return 0;
  return at::smallcache_tile_for_budget(d, m_elems);
}

int64_t attn_smallcache_onchip_elems(int64_t b) { return at::smallcache_onchip_elems(b); }

size_t attn_fwd_smallcache_workspace_size(int64_t bh, int64_t n, int64_t d, int64_t m_elems) {
  if (!shape_ok(bh, n, d)) return 0;
  const int64_t b = attn_smallcache_tile(d, m_elems);
  if (b == 0) return 0;
  return at::smallcache_workspace_bytes(bh, n, b);
}

attn_status attn_fwd_smallcache(const void* Q, const void* K, const void* V, float* O,
                                float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                attn_dtype dtype, int64_t m_elems, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (!at::smallcache_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (m_elems <= 0 || m_elems >= d * d) return ATTN_ERR_INVALID_ARG;
  const int64_t b = at::smallcache_tile_for_budget(d, m_elems);
  if (b == 0) return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  const size_t need = at::smallcache_workspace_bytes(bh, n, b);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned256(workspace)) return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_fwd_smallcache_bf16(Q, K, V, O, lse, bh, n, d, scale, b,
                                                      workspace,
                                                      static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_size(int64_t bh, int64_t n, int64_t d) {
  if (!shape_ok(bh, n, d) || !at::bwd_supported(d)) return 0;
  return at::bwd_workspace_bytes(bh, n, d);
}

int64_t attn_bwd_onchip_elems(int64_t d) { return at::bwd_onchip_elems(d); }

namespace {

attn_status bwd_checked(const char* tile, const void* Q, const void* K, const void* V,
                        const float* O, const void* dO, const float* lse, float* dQ, float* dK,
                        float* dV, int64_t bh, int64_t n, int64_t d, float scale,
                        attn_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (!at::bwd_supported(d) || at::bwd_tile_info(d, tile).keys_per_block == 0)
    return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  const size_t need = at::bwd_workspace_bytes(bh, n, d);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned256(workspace)))
    return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_bwd_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, bh, n, d, scale,
                                           workspace, tile, static_cast<hipStream_t>(stream)));
}

}  // namespace

attn_status attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                     const void* dO, const float* lse, float* dQ, float* dK, float* dV,
                     int64_t bh, int64_t n, int64_t d, float scale, attn_dtype dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_checked(nullptr, Q, K, V, O, dO, lse, dQ, dK, dV, bh, n, d, scale, dtype, workspace,
                     workspace_bytes, stream);
}

const char* attn_bwd_tiles(int64_t d) { return at::bwd_tile_names(d); }

attn_status attn_bwd_tile_info(const char* tile, int64_t d, int64_t* keys_per_block,
                               int64_t* queries_per_block, int64_t* key_tile,
                               int64_t* onchip_elems) {
  if (!tile) return ATTN_ERR_INVALID_ARG;
  const at::BwdTileInfo t = at::bwd_tile_info(d, tile);
  if (t.keys_per_block == 0) return ATTN_ERR_UNSUPPORTED;
  if (keys_per_block) *keys_per_block = t.keys_per_block;
  if (queries_per_block) *queries_per_block = t.queries_per_block;
  if (key_tile) *key_tile = t.key_tile;
  if (onchip_elems) *onchip_elems = t.onchip;
  return ATTN_OK;
}

attn_status attn_bwd_tile(const char* tile, const void* Q, const void* K, const void* V,
                          const float* O, const void* dO, const float* lse, float* dQ, float* dK,
                          float* dV, int64_t bh, int64_t n, int64_t d, float scale,
                          attn_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!tile) return ATTN_ERR_INVALID_ARG;
  return bwd_checked(tile, Q, K, V, O, dO, lse, dQ, dK, dV, bh, n, d, scale, dtype, workspace,
                     workspace_bytes, stream);
}

int64_t attn_bwd_smallcache_tile(int64_t d, int64_t m_elems) {
  return at::bwd_smallcache_tile(d, m_elems).b;
}

int64_t attn_bwd_smallcache_onchip_elems(int64_t d, int64_t m_elems) {
  const at::SmallBwdTile t = at::bwd_smallcache_tile(d, m_elems);
  return t.b ? at::bwd_smallcache_onchip_elems(t.b, t.stages) : 0;
}

size_t attn_bwd_smallcache_workspace_size(int64_t bh, int64_t n, int64_t d, int64_t m_elems) {
  if (!shape_ok(bh, n, d)) return 0;
  const at::SmallBwdTile t = at::bwd_smallcache_tile(d, m_elems);
  if (t.b == 0) return 0;
  return at::bwd_smallcache_workspace_bytes(bh, n, t.b);
}

attn_status attn_bwd_smallcache(const void* Q, const void* K, const void* V, const float* O,
                                const void* dO, const float* lse, float* dQ, float* dK,
                                float* dV, int64_t bh, int64_t n, int64_t d, float scale,
                                attn_dtype dtype, int64_t m_elems, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!shape_ok(bh, n, d) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (!at::bwd_smallcache_supported(d)) return ATTN_ERR_UNSUPPORTED;
  if (m_elems <= 0 || m_elems >= d * d) return ATTN_ERR_INVALID_ARG;
  const at::SmallBwdTile t = at::bwd_smallcache_tile(d, m_elems);
  if (t.b == 0) return ATTN_ERR_UNSUPPORTED;
  if (bh * n == 0) return ATTN_OK;
  // the n x n intermediates are indexed per head with 32-bit tile counts
  const int64_t nt = (n + t.b - 1) / t.b;
  if (nt * t.b > (int64_t(1) << 20) || bh * nt * nt >= (int64_t(1) << 31))
    return ATTN_ERR_INVALID_ARG;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  const size_t need = at::bwd_smallcache_workspace_bytes(bh, n, t.b);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return ATTN_ERR_WORKSPACE;
  return launch_status(at::launch_bwd_smallcache_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, bh, n, d,
                                                      scale, t, workspace,
                                                      static_cast<hipStream_t>(stream)));
}

attn_status attn_calib_mfma_loop(float* out, int64_t workgroups, int32_t iters, float amp,
                                 void* stream) {
  if (!out || !aligned16(out) || workgroups < 1 || workgroups > INT32_MAX || iters < 1 ||
      !std::isfinite(amp))
    return ATTN_ERR_INVALID_ARG;
  return launch_status(
      at::launch_calib_mfma_loop(out, workgroups, iters, amp, static_cast<hipStream_t>(stream)));
}

attn_status attn_calib_stream_read(const void* src, int64_t bytes, uint32_t* out,
                                   int64_t workgroups, void* stream) {
  if (!src || !aligned16(src) || bytes < 16 || bytes % 16 != 0 || !out || !aligned16(out) ||
      workgroups < 1 || workgroups > INT32_MAX / 256)
    return ATTN_ERR_INVALID_ARG;
  return launch_status(at::launch_calib_stream_read(src, bytes, out, workgroups,
                                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
