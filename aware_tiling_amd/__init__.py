"""Exact attention for MI355X (gfx950): fused streaming forward, square-tile
small-cache forward and backward, as hand-written HIP kernels behind a C ABI
(include/aware_tiling.h).  This package is the thin Python binding."""
from .binding import (SPARSE_BLOCK, AttnError, attn_bwd, attn_bwd_smallcache, attn_fwd,
                      attn_fwd_blocksparse, attn_fwd_budget, attn_fwd_smallcache,
                      attn_fwd_splitk, attn_fwd_splitk_noalloc, attn_fwd_tile, attn_bwd_tile,
                      bwd_onchip_elems, bwd_smallcache_tile, bwd_tile_info, bwd_tiles,
                      calib_mfma_loop, calib_stream_read,
                      default_scale, fwd_budget_onchip_elems, fwd_onchip_elems,
                      fwd_query_block, fwd_tile_info, fwd_tiles, lib, smallcache_tile,
                      splitk_splits)

__all__ = ["AttnError", "SPARSE_BLOCK", "attn_fwd", "attn_fwd_blocksparse", "attn_fwd_budget",
           "attn_fwd_splitk", "attn_fwd_splitk_noalloc", "attn_fwd_smallcache", "attn_fwd_tile", "attn_bwd",
           "attn_bwd_smallcache", "attn_bwd_tile", "bwd_onchip_elems", "bwd_smallcache_tile",
           "bwd_tile_info", "bwd_tiles", "calib_mfma_loop", "calib_stream_read",
           "default_scale",
           "fwd_budget_onchip_elems", "fwd_onchip_elems", "fwd_query_block", "fwd_tile_info",
           "fwd_tiles", "lib", "smallcache_tile", "splitk_splits"]
