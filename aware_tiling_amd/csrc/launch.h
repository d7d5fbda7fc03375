// Host-side launchers of the HIP kernels.  Arguments are validated by the
// C-ABI layer (api.cpp) before any of these is called; each launcher only
// enqueues kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace at {

// Tile configuration of the fused forward for one head dimension.
struct FusedTileInfo {
  int block_rows;    // B: query rows per workgroup
  int key_tile;      // keys per K/V tile
  int64_t onchip;    // elements held on chip per workgroup (M)
};

// bf16 tile shapes: `tile` names a compiled shape for d, nullptr the
// default one.  fused_bf16_tile_names(d) lists the names (default first,
// space separated; "" for an unsupported d).
bool fused_bf16_supported(int64_t d);
bool fused_f32_supported(int64_t d);
FusedTileInfo fused_bf16_tile_info(int64_t d, const char* tile = nullptr);
const char* fused_bf16_tile_names(int64_t d);
FusedTileInfo fused_f32_tile_info(int64_t d);

hipError_t launch_fwd_fused_bf16(const void* Q, const void* K, const void* V, float* O,
                                 float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                 const char* tile, hipStream_t stream);
// Fused forward with 32-row query blocks and 32-key tiles, four waves each
// owning a quarter of d (fwd_budget.hip): the fused schedule held to a
// budget below d^2.
bool fused_budget_supported(int64_t d);
int64_t fused_budget_onchip(int64_t d);
hipError_t launch_fwd_budget_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                  hipStream_t stream);
hipError_t launch_fwd_fused_f32(const float* Q, const float* K, const float* V, float* O,
                                float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                hipStream_t stream);

// Key-split forward for rectangular shapes (nq queries, nk keys per head).
// `splits` is the requested count (>= 1); the keys are cut into chunks of
// splitk_key_chunk() keys (a multiple of the 64-key tile), so the effective
// count can be smaller.  With one effective split the kernel writes O and lse
// directly and needs no workspace.
size_t align256_bytes(size_t b);
bool splitk_supported(int64_t d);
int64_t splitk_auto_splits(int64_t bh, int64_t nq, int64_t nk, int64_t d);
int64_t splitk_key_chunk(int64_t nk, int64_t splits);
int64_t splitk_effective_splits(int64_t nk, int64_t splits);
size_t splitk_workspace_bytes(int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t splits);
hipError_t launch_fwd_splitk_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t nq, int64_t nk, int64_t d,
                                  float scale, int64_t splits, void* workspace,
                                  hipStream_t stream);
// The same with the partials in the library's own device array of
// kSplitkScratchBytes (no workspace, no allocation); the caller checks
// splitk_workspace_bytes(...) <= kSplitkScratchBytes.
constexpr size_t kSplitkScratchBytes = size_t(16) << 20;
hipError_t launch_fwd_splitk_noalloc_bf16(const void* Q, const void* K, const void* V, float* O,
                                          float* lse, int64_t bh, int64_t nq, int64_t nk,
                                          int64_t d, float scale, int64_t splits,
                                          hipStream_t stream);

// Block-sparse forward: a byte mask [mask_heads][nb][nb] over square blocks
// of kSparseBlock queries x kSparseBlock keys (nb = ceil(n / kSparseBlock));
// mask_heads is 1 (shared) or bh.  The workspace holds per-row tile counts
// and tile lists.
constexpr int kSparseBlock = 128;
size_t sparse_workspace_bytes(int64_t n, int64_t mask_heads);
hipError_t launch_fwd_sparse_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                  const uint8_t* mask, int64_t mask_heads, void* workspace,
                                  hipStream_t stream);

// Square-tile (small-cache) forward.
bool smallcache_supported(int64_t d);
int64_t smallcache_tile_for_budget(int64_t d, int64_t m_elems);
int64_t smallcache_onchip_elems(int64_t b);
size_t smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b);
hipError_t launch_fwd_smallcache_bf16(const void* Q, const void* K, const void* V, float* O,
                                      float* lse, int64_t bh, int64_t n, int64_t d,
                                      float scale, int64_t b, void* workspace,
                                      hipStream_t stream);

// Backward.
bool bwd_supported(int64_t d);
// Blockwise backward tile shapes: keys per dK/dV workgroup, queries per dQ
// workgroup, keys per dQ tile, and on-chip elements (the larger kernel's).
struct BwdTileInfo {
  int keys_per_block, queries_per_block, key_tile;
  int64_t onchip;
};
// `tile` names a compiled shape for d (nullptr: the default); all zeros if
// unknown.  bwd_tile_names(d): the names, default first, space separated.
BwdTileInfo bwd_tile_info(int64_t d, const char* tile = nullptr);
const char* bwd_tile_names(int64_t d);
int64_t bwd_onchip_elems(int64_t d);  // the default shape's footprint
size_t bwd_workspace_bytes(int64_t bh, int64_t n, int64_t d);
hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const float* O,
                           const void* dO, const float* lse, float* dQ, float* dK, float* dV,
                           int64_t bh, int64_t n, int64_t d, float scale, void* workspace,
                           const char* tile, hipStream_t stream);

// D_i = <dO_i, O_i> for rows = bh * n rows of width d in {64, 128, 256}.
hipError_t launch_bwd_preprocess(const float* O, const void* dO, float* Dout, int64_t rows,
                                 int64_t d, hipStream_t stream);

// Square-tile (small-cache) backward.  The tile side b and the number of
// staged panels are chosen from the on-chip budget M (elements, M < d^2).
struct SmallBwdTile {
  int b;       // square tile side, 0 if none fits
  int stages;  // LDS panel stages (1 or 2)
};
bool bwd_smallcache_supported(int64_t d);
int64_t bwd_smallcache_onchip_elems(int64_t b, int64_t stages);
SmallBwdTile bwd_smallcache_tile(int64_t d, int64_t m_elems);
size_t bwd_smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b);
hipError_t launch_bwd_smallcache_bf16(const void* Q, const void* K, const void* V,
                                      const float* O, const void* dO, const float* lse,
                                      float* dQ, float* dK, float* dV, int64_t bh, int64_t n,
                                      int64_t d, float scale, SmallBwdTile t, void* workspace,
                                      hipStream_t stream);

// Matrix-core loop for the reachable bf16 MFMA rate (calib.hip).
hipError_t launch_calib_mfma_loop(float* out, int64_t workgroups, int iters, float amp,
                                  hipStream_t stream);
// Streaming read for the reachable HBM read bandwidth (calib.hip).
hipError_t launch_calib_stream_read(const void* src, int64_t bytes, uint32_t* out,
                                    int64_t workgroups, hipStream_t stream);

}  // namespace at
