// Integer index maps of the gfx950 attention kernels: LDS swizzles, the
// key order of transposed value reads, the workgroup -> tile remap, and the
// per-lane byte and element offsets of the tile copies and operand reads.
//
// Everything here is constexpr and free of device intrinsics, so the same
// definitions compile for the kernels (clang treats constexpr functions as
// usable on both sides) and for the host-side test that enumerates every
// lane, row, tile and stage and checks bounds and bijections
// (tests/index/index_check.cpp).
//
// Conventions: a tile is `rows` rows of D bf16 values, row-major, stored in
// LDS as 16-byte chunks (CPR = D / 8 per row).  LDS chunk p holds row
// p / CPR, physical chunk p % CPR, which carries logical chunk
// (p % CPR) ^ swizzle(row) of that row.
#pragma once

#include <stdint.h>

namespace at {

// XOR swizzle of the 16-byte chunk index inside an LDS row, chosen so that
// when consecutive rows are read at the same logical chunk (one row per
// lane), the lanes of one ds_read_b128 phase land on distinct banks, whether
// a phase spans 128 bytes (8 lanes) or 256 bytes (16 lanes).  Rows of 256
// bytes or more use the low four row bits; 128-byte rows alternate bank
// halves between even and odd rows, so they fold bit 3 into bit 0; 64-byte
// rows put four rows in 256 bytes and mix bits 1 and 2.
template <int ROW_BYTES>
constexpr int chunk_swizzle(int row) {
  static_assert(ROW_BYTES >= 64, "rows shorter than 64 bytes are not swizzled");
  if constexpr (ROW_BYTES >= 256)
    return row & 15;
  else if constexpr (ROW_BYTES == 128)
    return (row & 7) ^ ((row >> 3) & 1);
  else
    return ((row >> 1) ^ (row >> 2)) & 3;
}

// Swizzle of the 16-byte chunk index for a row-major value tile read with
// ds_read_b64_tr_b16 (rows of ROW_BYTES).  One such read touches 4
// consecutive rows at the same 4-chunk group per half wave; flipping bits 2-3
// of the chunk index by the row (d >= 128) or by row bit 1 (d = 64, two rows
// per 256 bytes) spreads those 4 rows over all 64 banks.
template <int ROW_BYTES>
constexpr int vtr_swizzle(int row) {
  if constexpr (ROW_BYTES >= 256)
    return 4 * (row & 3);
  else
    return 4 * ((row >> 1) & 1);
}

// Swizzle for a row-major tile that is read both ways: row-wise with
// ds_read_b128 (16 consecutive rows at one logical chunk per phase) and
// transposed with ds_read_b64_tr_b16 (4 consecutive rows x 4 consecutive
// chunks per half wave).  The XOR value is a bijection of the low 4 row bits
// (distinct for any 16 consecutive rows) whose bits 2-3 are the row's low
// bits (distinct 64-byte chunk groups for any 4 consecutive rows).  For
// 128-byte rows (two rows per 256-byte bank window) bit 2 follows row bit 1
// instead.
template <int ROW_BYTES>
constexpr int dual_swizzle(int row) {
  if constexpr (ROW_BYTES >= 256)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Position of key k inside a transposed value tile: within each group of 16
// keys, bits 2 and 3 of the key index are swapped, so that the 8 keys one
// lane feeds to the P*V product are contiguous.
constexpr int vt_key_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Map the hardware workgroup id to a logical tile id so that consecutive
// logical tiles run on the same XCD (workgroups are dispatched round robin
// over the 8 XCDs); tiles that share K/V then share that XCD's L2.
constexpr int xcd_remap(int w, int total) {
  const int per = total >> 3;
  if (w < (per << 3)) return (w & 7) * per + (w >> 3);
  return w;
}

// Tile copy: byte offset, within a row-major tile in global memory, of the
// 16 bytes that land in LDS chunk p (LDS byte offset 16 p): row p / CPR,
// logical chunk (p % CPR) ^ SWZ(row).
template <int D, int (*SWZ)(int)>
constexpr uint32_t tile_copy_src(int p) {
  const int row = p / (D / 8), phys = p % (D / 8);
  return (uint32_t)(row * D + (phys ^ SWZ(row)) * 8) * 2u;
}

// The logical chunk (within its row p / CPR) that LDS chunk p holds.
template <int D, int (*SWZ)(int)>
constexpr int tile_copy_chunk(int p) {
  return (p % (D / 8)) ^ SWZ(p / (D / 8));
}

// Element offset, within an LDS tile of D-wide rows, of logical 16-byte
// chunk `chunk` of row `row` (where the tile copy put it).
template <int D, int (*SWZ)(int)>
constexpr int row_chunk_elem(int row, int chunk) {
  return row * D + ((chunk ^ SWZ(row)) * 8);
}

// Element offset, within an LDS tile of D-wide rows, of logical element
// (row, col) (col % 8 <= 4 for a 4-element transposed read piece).
template <int D, int (*SWZ)(int)>
constexpr int tile_elem(int row, int col) {
  return row * D + (((col >> 3) ^ SWZ(row)) * 8) + (col & 7);
}

// Transposed operand reads (ds_read_b64_tr_b16) of a 32 x 16 A operand from
// a row-major tile, rows = the contraction index: within each group of 16
// lanes (G = lane / 16, s = lane % 16), source lane s points at tile row
// 8 piece + 4 (G / 2) + s / 4 of the 16-row step and at column
// 16 (G % 2) + 4 (s % 4) of the 32-column block, so that each lane receives
// one column across 4 consecutive rows and two pieces give the 8 k-slots in
// the score accumulator's row order.
constexpr int tr_read_row(int lane, int piece) {
  return 8 * piece + 4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2);
}
constexpr int tr_read_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

}  // namespace at
