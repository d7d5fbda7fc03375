// Host-side check of the gfx950 kernels' integer index maps
// (aware_tiling_amd/csrc/index_maps.h): every lane, row, tile and stage of
// the tile copies and operand reads the fused forward and the blockwise
// backward use, at the tile shapes the library compiles.
//
// Checked, for each shape:
//  - swizzles keep chunk indices in range, are bijections per row, repeat
//    every 16 rows (the backward adds whole 16- and 32-row steps to offsets
//    computed once), and give the bank-conflict-free phases their comments
//    state;
//  - the tile copy maps the LDS chunks one to one onto the tile's chunks,
//    inside the tile and the LDS buffer;
//  - every row-wise operand read lands inside the tile on the chunk the copy
//    put its (row, logical chunk) in;
//  - every transposed read (simulating ds_read_b64_tr_b16: within a group of
//    16 lanes, lane i receives element i % 4 of the 8 bytes addressed by
//    lanes 4 e + i / 4) gives lane l the column l % 32 of the 32-column block
//    across the 8 tile rows whose order matches the score accumulator's row
//    order for k-slots 8 (l / 32) .. + 7;
//  - vt_key_pos is a permutation, xcd_remap a permutation of the grid.
// Prints "index maps: N checks passed" and exits 0, or prints the first
// failure and exits 1.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "index_maps.h"

using namespace at;

static long g_checks = 0;

// CHECK(condition, printf-style message...): the condition is evaluated
// once; on failure the message and the line are printed and the program
// exits with status 1.  (Template argument lists in conditions need no
// extra parentheses: the arguments go to a function.)
static void check_at(int line, bool ok, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
static void check_at(int line, bool ok, const char* fmt, ...) {
  ++g_checks;
  if (ok) return;
  std::fprintf(stderr, "FAILED line %d: ", line);
  va_list ap;
  va_start(ap, fmt);
  std::vfprintf(stderr, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "\n");
  std::exit(1);
}
#define CHECK(...) check_at(__LINE__, __VA_ARGS__)

// Bank group (16-byte unit of the 64 x 4-byte bank window) of an LDS byte
// offset.
static int bank16(long byte) { return (int)((byte / 16) % 16); }

template <int ROW_BYTES, int (*SWZ)(int)>
static void check_swizzle_basic(const char* name) {
  constexpr int CPR = ROW_BYTES / 16;
  for (int row = 0; row < 1024; ++row) {
    const int s = SWZ(row);
    CHECK(s >= 0 && s < CPR, "%s<%d>(%d) = %d out of [0, %d)", name, ROW_BYTES, row, s, CPR);
    CHECK(SWZ(row + 16) == s, "%s<%d> not periodic in 16 rows at row %d", name, ROW_BYTES, row);
    std::set<int> seen;
    for (int c = 0; c < CPR; ++c) seen.insert(c ^ s);
    CHECK((int)seen.size() == CPR && *seen.rbegin() == CPR - 1, "%s<%d> row %d not a bijection",
          name, ROW_BYTES, row);
  }
}

// Row-wise reads: `lanes` consecutive rows (one per lane) at one logical
// chunk occupy distinct 16-byte bank groups.
template <int ROW_BYTES, int (*SWZ)(int)>
static void check_rowwise_phase(const char* name, int lanes) {
  constexpr int CPR = ROW_BYTES / 16;
  for (int r0 = 0; r0 < 64; r0 += lanes)
    for (int c = 0; c < CPR; ++c) {
      std::set<int> banks;
      for (int i = 0; i < lanes; ++i) {
        const int row = r0 + i;
        banks.insert(bank16((long)row * ROW_BYTES + (long)(c ^ SWZ(row)) * 16));
      }
      CHECK((int)banks.size() == lanes, "%s<%d>: rows %d..+%d at chunk %d share banks", name,
            ROW_BYTES, r0, lanes - 1, c);
    }
}

// Transposed reads: 4 consecutive rows x a group of 4 consecutive chunks
// (the 16 chunks one half-wave's ds_read_b64_tr_b16 touches) occupy
// distinct 16-byte bank groups.
template <int ROW_BYTES, int (*SWZ)(int)>
static void check_tr_phase(const char* name) {
  constexpr int CPR = ROW_BYTES / 16;
  if (CPR < 4) return;
  for (int r0 = 0; r0 < 64; r0 += 4)
    for (int c0 = 0; c0 < CPR; c0 += 4) {
      std::set<int> banks;
      for (int e = 0; e < 4; ++e)
        for (int c = c0; c < c0 + 4; ++c)
          banks.insert(bank16((long)(r0 + e) * ROW_BYTES + (long)(c ^ SWZ(r0 + e)) * 16));
      CHECK((int)banks.size() == 16, "%s<%d>: rows %d..+3 x chunks %d..+3 share banks", name,
            ROW_BYTES, r0, c0);
    }
}

// Tile copy of a tile of `rows` rows, `nw` waves, `insts` copies per wave:
// lane chunk p = wave * (chunks / nw) + it * 64 + lane.
template <int D, int (*SWZ)(int)>
static void check_copy(const char* what, int rows, int nw) {
  const int cpr = D / 8, chunks = rows * cpr;
  CHECK(chunks % (nw * 64) == 0, "%s: %d chunks do not split into %d whole waves", what, chunks,
        nw);
  const int wave_chunks = chunks / nw, insts = wave_chunks / 64;
  std::vector<int> hit(chunks, 0);
  for (int w = 0; w < nw; ++w)
    for (int it = 0; it < insts; ++it)
      for (int lane = 0; lane < 64; ++lane) {
        const int p = w * wave_chunks + it * 64 + lane;
        CHECK(p >= 0 && p < chunks, "%s: LDS chunk %d outside the tile", what, p);
        const uint32_t src = tile_copy_src<D, SWZ>(p);
        CHECK(src % 16 == 0 && src < (uint32_t)rows * D * 2, "%s: source offset %u outside", what,
              src);
        const int row = p / cpr, chunk = tile_copy_chunk<D, SWZ>(p);
        CHECK(src == (uint32_t)(row * D + chunk * 8) * 2u, "%s: chunk %d source mismatch", what, p);
        hit[src / 16]++;
      }
  for (int c = 0; c < chunks; ++c) CHECK(hit[c] == 1, "%s: source chunk %d copied %d times", what, c, hit[c]);
}

// Row-wise operand read of logical chunk `chunk` of tile row `row` lands on
// the LDS chunk holding it.
template <int D, int (*SWZ)(int)>
static void check_row_read(const char* what, int rows) {
  for (int row = 0; row < rows; ++row)
    for (int chunk = 0; chunk < D / 8; ++chunk) {
      const int e = row_chunk_elem<D, SWZ>(row, chunk);
      CHECK(e % 8 == 0 && e >= 0 && e < rows * D, "%s: row %d chunk %d at %d outside", what, row,
            chunk, e);
      const int p = e / 8;
      CHECK(p / (D / 8) == row && tile_copy_chunk<D, SWZ>(p) == chunk,
            "%s: row %d chunk %d reads LDS chunk %d holding another", what, row, chunk, p);
    }
}

// Transposed read of a 32 x 16 A operand (32 columns of block `db` x 16 tile
// rows from `row0`), simulated per lane; element j of lane l's operand must
// be tile (row0 + 8 (j / 4) + 4 (l / 32) + j % 4, 32 db + l % 32).
template <int D, int (*SWZ)(int)>
static void check_tr_read(const char* what, int rows, int row0, int db) {
  long addr[64];  // element offset each lane points at, per piece
  for (int piece = 0; piece < 2; ++piece) {
    for (int lane = 0; lane < 64; ++lane) {
      const int row = row0 + tr_read_row(lane, piece), col = db * 32 + tr_read_col(lane);
      const int e = tile_elem<D, SWZ>(row, col);
      CHECK(e >= 0 && e + 4 <= rows * D, "%s: lane %d piece %d reads outside", what, lane, piece);
      CHECK(e / 8 == (e + 3) / 8, "%s: lane %d piece %d straddles chunks", what, lane, piece);
      addr[lane] = e;
    }
    for (int lane = 0; lane < 64; ++lane) {
      const int g = lane & ~15, i = lane & 15;
      for (int el = 0; el < 4; ++el) {
        const long src = addr[g + 4 * el + i / 4] + (i % 4);  // element received
        const int p = (int)(src / 8), row = p / (D / 8);
        const int col = tile_copy_chunk<D, SWZ>(p) * 8 + (int)(src % 8);
        const int j = 4 * piece + el;
        const int want_row = row0 + 8 * (j / 4) + 4 * (lane / 32) + j % 4;
        const int want_col = db * 32 + lane % 32;
        CHECK(row == want_row && col == want_col,
              "%s: lane %d k-slot %d gets (%d, %d), wants (%d, %d)", what, lane, j, row, col,
              want_row, want_col);
      }
    }
  }
}

template <int D, int NW, int BC>
static void check_fused_forward(const char* name) {
  // K tile: copy with chunk_swizzle, row-wise reads (rows kb * 32 + li).
  check_copy<D, chunk_swizzle<D * 2>>(name, BC, NW);
  check_row_read<D, chunk_swizzle<D * 2>>(name, BC);
  // V tile: copy with vtr_swizzle, transposed reads per (32-key block,
  // 16-key half, 32-column block).
  check_copy<D, vtr_swizzle<D * 2>>(name, BC, NW);
  for (int kb = 0; kb < BC / 32; ++kb)
    for (int half = 0; half < 2; ++half)
      for (int db = 0; db < D / 32; ++db)
        check_tr_read<D, vtr_swizzle<D * 2>>(name, BC, kb * 32 + 16 * half, db);
  // LDS: two K and two V tiles of BC x D bf16 within 160 KiB.
  CHECK(4 * BC * D * 2 <= 160 * 1024, "%s: LDS %d bytes", name, 4 * BC * D * 2);
}

template <int D, int NW>
static void check_backward() {
  // dK/dV kernel: query tiles of BQ rows (whole-wave copies), dual swizzle,
  // row reads at rows li + 32 qb (offsets computed at li, whole rows added),
  // transposed reads per 16-row step.
  constexpr int BQ = (32 * D / 8) % (NW * 64) == 0 ? 32 : 64;
  check_copy<D, dual_swizzle<D * 2>>("bwd dK/dV Q/dO tile", BQ, NW);
  check_row_read<D, dual_swizzle<D * 2>>("bwd Q/dO rows", BQ);
  for (int li = 0; li < 32; ++li)
    for (int qb = 0; qb < BQ / 32; ++qb)
      for (int chunk = 0; chunk < D / 8; ++chunk)
        CHECK(row_chunk_elem<D, dual_swizzle<D * 2>>(li, chunk) + qb * 32 * D ==
                  row_chunk_elem<D, dual_swizzle<D * 2>>(li + 32 * qb, chunk),
              "bwd: row %d + 32 x %d is not a whole-row step", li, qb);
  for (int ks = 0; ks < BQ / 16; ++ks)
    for (int db = 0; db < D / 32; ++db) {
      check_tr_read<D, dual_swizzle<D * 2>>("bwd Q^T/dO^T", BQ, 16 * ks, db);
      for (int lane = 0; lane < 64; ++lane)
        for (int piece = 0; piece < 2; ++piece)
          CHECK(tile_elem<D, dual_swizzle<D * 2>>(tr_read_row(lane, piece),
                                                   db * 32 + tr_read_col(lane)) +
                        16 * ks * D ==
                    tile_elem<D, dual_swizzle<D * 2>>(16 * ks + tr_read_row(lane, piece),
                                                      db * 32 + tr_read_col(lane)),
                "bwd: transposed read at step %d is not a whole-row step", ks);
    }
  // the wave's 32 V rows (copied with the dual swizzle, read row-wise)
  check_copy<D, dual_swizzle<D * 2>>("bwd V rows", 32, 1);
  // dQ kernel: 64-key K (dual) and V (row swizzle) tiles
  check_copy<D, dual_swizzle<D * 2>>("bwd dQ K tile", 64, NW);
  check_copy<D, chunk_swizzle<D * 2>>("bwd dQ V tile", 64, NW);
  check_row_read<D, dual_swizzle<D * 2>>("bwd dQ K rows", 64);
  check_row_read<D, chunk_swizzle<D * 2>>("bwd dQ V rows", 64);
  for (int ks = 0; ks < 4; ++ks)
    for (int db = 0; db < D / 32; ++db) check_tr_read<D, dual_swizzle<D * 2>>("bwd dQ K^T", 64, 16 * ks, db);
}

int main() {
  check_swizzle_basic<64, chunk_swizzle<64>>("chunk_swizzle");
  check_swizzle_basic<128, chunk_swizzle<128>>("chunk_swizzle");
  check_swizzle_basic<256, chunk_swizzle<256>>("chunk_swizzle");
  check_swizzle_basic<512, chunk_swizzle<512>>("chunk_swizzle");
  check_swizzle_basic<128, vtr_swizzle<128>>("vtr_swizzle");
  check_swizzle_basic<256, vtr_swizzle<256>>("vtr_swizzle");
  check_swizzle_basic<512, vtr_swizzle<512>>("vtr_swizzle");
  check_swizzle_basic<128, dual_swizzle<128>>("dual_swizzle");
  check_swizzle_basic<256, dual_swizzle<256>>("dual_swizzle");
  check_swizzle_basic<512, dual_swizzle<512>>("dual_swizzle");
  // row-wise phases: 16 lanes (256 bytes) and 8 lanes (128 bytes)
  check_rowwise_phase<128, chunk_swizzle<128>>("chunk_swizzle", 8);
  check_rowwise_phase<256, chunk_swizzle<256>>("chunk_swizzle", 16);
  check_rowwise_phase<512, chunk_swizzle<512>>("chunk_swizzle", 16);
  check_rowwise_phase<256, dual_swizzle<256>>("dual_swizzle", 16);
  check_rowwise_phase<512, dual_swizzle<512>>("dual_swizzle", 16);
  check_tr_phase<256, vtr_swizzle<256>>("vtr_swizzle");
  check_tr_phase<512, vtr_swizzle<512>>("vtr_swizzle");
  check_tr_phase<256, dual_swizzle<256>>("dual_swizzle");
  check_tr_phase<512, dual_swizzle<512>>("dual_swizzle");

  std::set<int> pos;
  for (int k = 0; k < 64; ++k) {
    const int v = vt_key_pos(k);
    CHECK(v / 16 == k / 16, "vt_key_pos(%d) = %d leaves its group of 16", k, v);
    pos.insert(v);
  }
  CHECK(pos.size() == 64, "vt_key_pos is not a permutation of 0..63");

  std::vector<int> totals;
  for (int t = 1; t <= 3000; ++t) totals.push_back(t);
  for (int t : {4096, 8192, 65536, 131072, 1 << 20}) totals.push_back(t);
  for (int total : totals) {
    std::vector<char> seen(total, 0);
    for (int w = 0; w < total; ++w) {
      const int t = xcd_remap(w, total);
      CHECK(t >= 0 && t < total && !seen[t], "xcd_remap(%d, %d) = %d repeats or leaves the grid",
            w, total, t);
      seen[t] = 1;
    }
  }

  // the fused forward's compiled shapes (head dimension, waves, keys per tile)
  check_fused_forward<128, 8, 64>("fwd d128 8x64");
  check_fused_forward<128, 2, 32>("fwd d128 2x32");
  check_fused_forward<128, 2, 64>("fwd d128 2x64");
  check_fused_forward<128, 4, 32>("fwd d128 4x32");
  check_fused_forward<128, 4, 64>("fwd d128 4x64");
  check_fused_forward<128, 8, 32>("fwd d128 8x32");
  check_fused_forward<256, 4, 32>("fwd d256 4x32");
  check_fused_forward<64, 8, 64>("fwd d64 8x64");
  check_fused_forward<64, 4, 64>("fwd d64 4x64 (split, sparse)");
  check_fused_forward<128, 4, 64>("fwd d128 4x64 (split, sparse)");
  check_fused_forward<64, 1, 32>("fwd d64 1x32 (decoding split)");
  check_fused_forward<128, 1, 32>("fwd d128 1x32 (decoding split)");
  check_backward<128, 8>();
  check_backward<64, 8>();
  check_backward<256, 4>();

  std::printf("index maps: %ld checks passed\n", g_checks);
  return 0;
}
