// Backward of exact attention for gfx950: dQ, dK, dV from Q, K, V, the
// forward's O and log-sum-exp, and the upstream gradient dO.
//
// Method: the page "On Fine-Grained I/O Complexity of Attention Backward
// Passes" (explainer), sections "Methodology" and "Key Contributions and
// Results" (Theorem 1.1), states the backward problem and that the blockwise
// large-cache schedule is optimal for M >= d^2; it prints no formulas.  The
// formulas are the exact derivatives of O = softmax(scale Q K^T) V:
//     P = exp(scale Q K^T - lse),   dV = P^T dO,   dP = dO V^T,
//     D_i = <dO_i, O_i> (= sum_j P_ij dP_ij),   dS = P o (dP - D),
//     dQ = scale dS K,   dK = scale dS^T Q.
// P is recomputed tile by tile from Q, K and the saved lse; no N x N matrix
// is stored.
//
// Three kernels, stream ordered:
//  1. bwd_preprocess: D_i = <dO_i, O_i> and lse_i log2(e) into the
//     workspace.
//  2. bwd_dkdv3: one workgroup per (head, block of 256 keys; 128 at
//     d = 256), one wave per 32 keys.  Each wave keeps its K rows as MFMA B operands and the
//     transposed accumulators dK^T, dV^T (d x 32 keys) in registers, its V
//     rows in LDS, and streams query tiles of Q, dO, lse, D through
//     double-buffered LDS.  Scores are computed as S = Q K^T so that a lane
//     owns one key: the bf16 P and dS tiles then feed dV^T += dO^T P and
//     dK^T += Q^T dS straight from registers, with Q^T and dO^T read from
//     the same row-major LDS tiles by transposing reads.
//  3. bwd_dq3: one workgroup per (head, block of 256 queries; 128 at
//     d = 256), one wave per 32 queries.  Each wave keeps Q and dO as B operands, lse and D as
//     per-lane scalars, and dQ^T in registers, and streams 64-key tiles of
//     K and V through LDS: S^T = K Q^T, dP^T = V dO^T, dS^T, and
//     dQ^T += K^T dS^T with K^T read transposed.  Recomputing S and dP here
//     costs 4 N^2 d more flops than accumulating dQ with atomics, and keeps
//     the result deterministic.
// At d = 256 the gradients' 1 KB rows leave through LDS (store_rows_lds),
// so that every store instruction writes whole rows.
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace at {

namespace {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. D_i = <dO_i, O_i>

// Also writes lse2 = lse log2(e) (the exponent base of the kernels) when
// lse2 is non-null.
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess(const float* __restrict__ O,
                                                      const bf16* __restrict__ dO,
                                                      float* __restrict__ Dout, int64_t rows,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ lse2) {
  constexpr int TPR = D / 8;       // threads per row (8 elements each)
  constexpr int RPB = 256 / TPR;   // rows per block
  const int t = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * RPB + t / TPR;
  const int c = (t % TPR) * 8;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * D + c);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + r * D + c);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + r * D + c + 4);
    acc = bf_lo(g[0]) * o0[0] + bf_hi(g[0]) * o0[1] + bf_lo(g[1]) * o0[2] + bf_hi(g[1]) * o0[3] +
          bf_lo(g[2]) * o1[0] + bf_hi(g[2]) * o1[1] + bf_lo(g[3]) * o1[2] + bf_hi(g[3]) * o1[3];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (r < rows && (t % TPR) == 0) {
    Dout[r] = acc;
    if (lse2 != nullptr) lse2[r] = lse[r] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK/dV and dQ kernels.  Tiles of Q and dO (dK/dV kernel) and of K and V
// (dQ kernel) go global -> LDS with buffer_load_dwordx4 ... lds and stay
// row-major.  These copies are issued from inline assembly, so that the
// next tile's copies stay in flight while the current tile is read (with
// compiler-visible copies in flight every wait for an LDS read becomes
// lgkmcnt(0)) and are waited for only at the end of the step.  They go
// through a buffer resource whose range ends at the head's last row, with
// the tile start as a scalar offset: one code path for every tile, and rows
// past n land as zeros, which the kernels give zero weight (lse = +inf for
// queries, an explicit mask for keys).  The transposed operands (Q^T,
// dO^T, K^T) come from ds_read_b64_tr_b16 on the same tiles, whose swizzle
// (dual_swizzle) keeps both the row-wise and the transposed reads free of
// bank conflicts.  No staging registers and no vector-ALU transposition, so
// two waves fit per SIMD at d <= 128.

namespace {

// Transposed A operand (32 rows of the d dimension x 16 rows of the tile)
// from a row-major dual-swizzled tile: k-slots follow the score
// accumulator's row order (tile rows 16 ks + 8 (j/4) + 4 h + j%4).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int ks, int db, int lane) {
  u32x2 part[2];
#pragma unroll
  for (int piece = 0; piece < 2; ++piece)
    part[piece] = lds_read_tr16(tile + tile_elem<D, dual_swizzle<D * 2>>(
                                           16 * ks + tr_read_row(lane, piece),
                                           db * 32 + tr_read_col(lane)));
  return __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
}

// Stores 32 rows of D fp32 accumulators, times `mul`, whose lane (li, h)
// holds row li, columns 32 db + 8 g + 4 h .. +3 in acc[db][4 g ..], through
// the wave's LDS region `st` (32 rows of D / 4 16-byte chunks, chunk c of row
// r at c ^ r), so that every store instruction writes whole rows; rows at or
// past `rows` are not stored.  The caller has finished with that LDS.
template <int D>
__device__ __forceinline__ void store_rows_lds(const f32x16 (&acc)[D / 32], float mul, f32x4* st,
                                               float* dst, int rows, int lane) {
  constexpr int CPR = D / 4;
  const int li = lane & 31, h = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = db * 8 + 2 * g + h;
      st[li * CPR + (c ^ li)] = f32x4{acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul,
                                      acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul};
    }
#pragma unroll
  for (int it = 0; it < 32 * CPR / 64; ++it) {
    const int idx = it * 64 + lane, r = idx / CPR, c = idx % CPR;
    const f32x4 v = st[r * CPR + (c ^ r)];
    if (r < rows) *reinterpret_cast<f32x4*>(dst + (size_t)r * D + c * 4) = v;
  }
}

template <int D>
__device__ __forceinline__ bf16x8 row_operand(const bf16* tile, int row, int chunk, bool dual) {
  return *reinterpret_cast<const bf16x8*>(
      tile + (dual ? row_chunk_elem<D, dual_swizzle<D * 2>>(row, chunk)
                   : row_chunk_elem<D, chunk_swizzle<D * 2>>(row, chunk)));
}

}  // namespace

template <int D, int NW>
struct DkdvCfg {
  static constexpr int NT = NW * 64, BKV = NW * 32;
  static constexpr int BQ = (32 * D / 8) % (NW * 64) == 0 ? 32 : 64;  // whole-wave loads
  static constexpr int CHUNKS = BQ * D / 8;
  static constexpr int WAVE_CHUNKS = CHUNKS / NW;
  static constexpr int INSTS = WAVE_CHUNKS / 64;
  static constexpr int TILE = BQ * D;
  // on-chip elements of one workgroup, each counted once whatever its width
  // and every pipeline slot counted (as for the forward): the K and V rows,
  // the dK^T and dV^T accumulators, both stages of the Q and dO tiles and of
  // their lse and D values, and the S/P and dP/dS tiles of all waves
  static constexpr int64_t ONCHIP =
      4 * (int64_t)BKV * D + 4 * (int64_t)BQ * D + 4 * BQ + 2 * (int64_t)BKV * BQ;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
};

// dK/dV kernel: one workgroup per block of NW * 32 keys, one wave per 32
// keys.  The wave keeps its K rows in registers (the B operand of S^T) and
// its V rows in LDS, and streams Q and dO tiles through LDS; per 32 queries
// it forms S = Q K^T, P = exp(S - lse), dV^T += dO^T P, dP = dO V^T,
// dS = P o (dP - D) and dK^T += Q^T dS.  Every LDS address is fixed before
// the loop: each lane's byte offsets into a tile (row-wise reads per
// k-step, transposed reads per 32-column block and half) are computed once,
// since the dual swizzle mixes only the low four bits of a row, which the
// lane fixes; the query sub-block, the k-step of the transposed reads and
// the tile (Q, dO, or the wave's V rows, stored with the same swizzle) only
// add constants, and the step is unrolled by two so that the stage is a
// constant as well.  Operands are read two MFMAs ahead.  The products are
// issued S, dP, dV, dK, so that the exponentials overlap the dP MFMAs and
// dS the dV MFMAs.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, (D >= 256 ? 1 : 8 / NW)) void bwd_dkdv3(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ Dg,
    float* __restrict__ dK, float* __restrict__ dV, int n, int nkb, int total, float c,
    float scale) {
  using C = DkdvCfg<D, NW>;
  constexpr int BQ = C::BQ;
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int TILE_B = C::TILE * 2;               // bytes of one Q or dO tile
  constexpr int VT_B = NW * 32 * D * 2;             // bytes of the V rows
  // [stage][Q | dO] tiles first (so every tile offset fits a read's
  // immediate), then the waves' V rows, then [stage][lse2 | D].
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_B + VT_B + 2 * 2 * BQ * 4];
  char* const tiles = smem;
  bf16* const vtile = reinterpret_cast<bf16*>(smem + 4 * TILE_B);
  float* const stats = reinterpret_cast<float*>(smem + 4 * TILE_B + VT_B);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / nkb, kblk = tile - head * nkb;
  const size_t hoff = (size_t)head * n * D;
  const bf16 *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff, *dOh = dO + hoff;
  const float* lseh = lse2 + (size_t)head * n;
  const float* Dh = Dg + (size_t)head * n;
  const int key = kblk * C::BKV + wave * 32 + li;

  // K rows of the wave's 32 keys in registers (zero past n); V rows in the
  // wave's LDS region (clamped to n-1): only the unstored dK/dV rows of
  // keys past n see either.
  bf16* const Vw = vtile + wave * 32 * D;
  bf16x8 kreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    kreg[kk] = key < n ? *reinterpret_cast<const bf16x8*>(Kh + (size_t)key * D + 16 * kk + 8 * h)
                       : bf16x8{};
  {
    constexpr int RC = D / 8;
#pragma unroll
    for (int it = 0; it < 32 * RC / 64; ++it) {
      const int p = it * 64 + lane;
      const int logical = tile_copy_chunk<D, dual_swizzle<D * 2>>(p);
      const int vrow = min(kblk * C::BKV + wave * 32 + p / RC, n - 1);
      load_lds_16(Vh + (size_t)vrow * D + logical * 8, Vw + it * 64 * 8);
    }
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = f32x16{};

  // Copy offsets (global side) and read offsets (LDS side), per lane.
  uint32_t toff[C::INSTS];
#pragma unroll
  for (int it = 0; it < C::INSTS; ++it) {
    toff[it] = tile_copy_src<D, dual_swizzle<D * 2>>(wave * C::WAVE_CHUNKS + it * 64 + lane);
  }
  // roff: row-wise reads of Q, dO and the wave's V rows (one swizzle);
  // troff: transposed reads.  The dual swizzle depends only on the low four
  // row bits, so further rows (query sub-block, k-step) add whole rows.
  uint32_t roff[NKK], troff[NDB][2];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    roff[kk] = (uint32_t)row_chunk_elem<D, dual_swizzle<D * 2>>(li, 2 * kk + h) * 2u;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int piece = 0; piece < 2; ++piece)
      troff[db][piece] = (uint32_t)tile_elem<D, dual_swizzle<D * 2>>(
                             tr_read_row(lane, piece), db * 32 + tr_read_col(lane)) * 2u;

  // Q and dO tiles through buffer resources over the head's n rows: rows
  // past n land as zeros (and get lse = +inf below, so weight 0).
  const rsrc_t rsQ = buffer_rsrc(Qh, (uint32_t)n * (D * 2));
  const rsrc_t rsG = buffer_rsrc(dOh, (uint32_t)n * (D * 2));
  const uint32_t tiles_lds = lds_addr(tiles);
  auto load = [&](int i, int stage) {
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(i * BQ) * (D * 2);
    const uint32_t ql = tiles_lds + stage * 2 * TILE_B;
#pragma unroll
    for (int it = 0; it < C::INSTS; ++it) {
      const uint32_t p0 = (uint32_t)(wave * C::WAVE_CHUNKS + it * 64) * 16;
      dma16_buf_at(rsQ, toff[it], so, ql + p0);
      dma16_buf_at(rsG, toff[it], so, ql + TILE_B + p0);
    }
    if (wave * 64 < 2 * BQ) {  // whole waves: 2 BQ is a multiple of 64
      // A query row past n (zeros in the Q and dO tiles) gets lse2 = +inf,
      // so its weights are exactly 0; its D stays finite.
      float* st = stats + stage * 2 * BQ;
      const int which = tid / BQ, r = tid - which * BQ;
      const int qrow = min(i * BQ + r, n - 1);
      if (which == 0 && i * BQ + r >= n)
        st[tid] = __builtin_inff();
      else
        dma4((which == 0 ? lseh : Dh) + qrow, st + wave * 64);
    }
  };

  const int nqt = (n + BQ - 1) / BQ;
  auto step = [&](auto stage_c, int i) {
    constexpr int P = decltype(stage_c)::value;
    if (i + 1 < nqt) load(i + 1, P ^ 1);
    const char* Qs = tiles + P * 2 * TILE_B;
    const char* Gs = Qs + TILE_B;
    const float* st = stats + P * 2 * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      constexpr int NA = 2 * NKK + 4 * NDB, AH = 2;
      bf16x8 a[NA];
      auto row_rd = [&](const char* t, int kk) {
        return *reinterpret_cast<const bf16x8*>(t + roff[kk] + qb * 32 * D * 2);
      };
      auto tr_rd = [&](const char* t, int ksp, int db) {
        const u32x2 p0 =
            lds_read_tr16(reinterpret_cast<const bf16*>(t + troff[db][0] + ksp * 16 * D * 2));
        const u32x2 p1 =
            lds_read_tr16(reinterpret_cast<const bf16*>(t + troff[db][1] + ksp * 16 * D * 2));
        return __builtin_bit_cast(bf16x8, (u32x4{p0[0], p0[1], p1[0], p1[1]}));
      };
      // operand sequence: S (Q rows), dP (dO rows), dV (dO^T), dK (Q^T)
      constexpr int T_DP = NKK, T_DV = 2 * NKK;
      constexpr int T_DK = 2 * NKK + 2 * NDB;
      auto fetch = [&](int t) {
        if (t < NKK) {
          a[t] = row_rd(Qs, t);
        } else if (t >= T_DV && t < T_DV + 2 * NDB) {
          const int u = t - T_DV;
          a[t] = tr_rd(Gs, 2 * qb + u / NDB, u % NDB);
        } else if (t >= T_DP && t < T_DP + NKK) {
          a[t] = row_rd(Gs, t - T_DP);
        } else {
          const int u = t - T_DK;
          a[t] = tr_rd(Qs, 2 * qb + u / NDB, u % NDB);
        }
      };
      auto use = [&](int t) -> bf16x8 {
        if (t + AH < NA) fetch(t + AH);
        return a[t];
      };
#pragma unroll
      for (int t = 0; t < AH; ++t) fetch(t);
      // the compiler's exponential/MFMA interleaving strategy for this
      // block (1.6 % faster at d = 128, 5 % at d = 256, the same bits; at
      // d = 128 it costs one spilled register, reloaded only on the path
      // that marks query rows past n)
      if constexpr (D >= 128) __builtin_amdgcn_iglp_opt(3);
      // S = Q K^T, P = 2^(S c - lse2) in bf16, dV^T += dO^T P; dP = dO V^T,
      // dS = P o (dP - D) from the same bf16 P, dK^T += Q^T dS.  The dP
      // MFMAs follow the S MFMAs directly, so the exponentials run while
      // they execute and dS while the dV MFMAs do (two score-sized
      // accumulators live instead of one).
      f32x16 s = {}, dp = {};
      uint32_t pk[8];
      auto scores = [&]() {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) s = mfma_bf16_32x32x16(use(kk), kreg[kk], s);
      };
      auto exps = [&]() {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(st + qb * 32 + 8 * g + 4 * h);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = fast_exp2(__builtin_fmaf(s[4 * g + e], c, -l2[e]));
          pk[2 * g] = pack_bf16x2(p[0], p[1]);
          pk[2 * g + 1] = pack_bf16x2(p[2], p[3]);
        }
      };
      auto dv_update = [&]() {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 bp = __builtin_bit_cast(
              bf16x8, (u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]}));
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dvt[db] = mfma_bf16_32x32x16(use(T_DV + ks * NDB + db), bp, dvt[db]);
        }
      };
      auto dprod = [&]() {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 vb =
              *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(Vw) + roff[kk]);
          dp = mfma_bf16_32x32x16(use(T_DP + kk), vb, dp);
        }
      };
      scores();
      dprod();
      exps();
      dv_update();
      uint32_t dsk[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 dd = *reinterpret_cast<const f32x4*>(st + BQ + qb * 32 + 8 * g + 4 * h);
        const float p0 = bf_lo(pk[2 * g]), p1 = bf_hi(pk[2 * g]);
        const float p2 = bf_lo(pk[2 * g + 1]), p3 = bf_hi(pk[2 * g + 1]);
        dsk[2 * g] = pack_bf16x2(p0 * (dp[4 * g] - dd[0]), p1 * (dp[4 * g + 1] - dd[1]));
        dsk[2 * g + 1] = pack_bf16x2(p2 * (dp[4 * g + 2] - dd[2]), p3 * (dp[4 * g + 3] - dd[3]));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bs = __builtin_bit_cast(
            bf16x8, (u32x4{dsk[4 * ks], dsk[4 * ks + 1], dsk[4 * ks + 2], dsk[4 * ks + 3]}));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dkt[db] = mfma_bf16_32x32x16(use(T_DK + ks * NDB + db), bs, dkt[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's copies, before the barrier
    __syncthreads();
  };

  load(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int i = 0;
  for (; i + 1 < nqt; i += 2) {
    step(std::integral_constant<int, 0>{}, i);
    step(std::integral_constant<int, 1>{}, i + 1);
  }
  if (i < nqt) step(std::integral_constant<int, 0>{}, i);

  if constexpr (D >= 256) {
    // 1 KB rows leave through LDS (whole rows per store instruction)
    __syncthreads();  // every wave is done with the tiles, V rows and stats
    f32x4* const st = reinterpret_cast<f32x4*>(smem) + wave * 32 * (D / 4);
    const int k0 = kblk * C::BKV + wave * 32;
    store_rows_lds<D>(dkt, scale, st, dK + hoff + (size_t)k0 * D, n - k0, lane);
    store_rows_lds<D>(dvt, 1.f, st, dV + hoff + (size_t)k0 * D, n - k0, lane);
  } else if (key < n) {
    float* dKr = dK + hoff + (size_t)key * D;
    float* dVr = dV + hoff + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = db * 32 + 8 * g + 4 * h;
        f32x4 a = {dkt[db][4 * g] * scale, dkt[db][4 * g + 1] * scale, dkt[db][4 * g + 2] * scale,
                   dkt[db][4 * g + 3] * scale};
        f32x4 b = {dvt[db][4 * g], dvt[db][4 * g + 1], dvt[db][4 * g + 2], dvt[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dKr + col) = a;
        *reinterpret_cast<f32x4*>(dVr + col) = b;
      }
  }
}

template <int D, int NW, int BC>
struct DqCfg {
  static constexpr int NT = NW * 64, BQB = NW * 32;
  static constexpr int CHUNKS = BC * D / 8;
  static constexpr int WAVE_CHUNKS = CHUNKS / NW;
  static constexpr int INSTS = WAVE_CHUNKS / 64;
  static constexpr int TILE = BC * D;
  // on-chip elements (as DkdvCfg): the Q and dO rows, the dQ^T accumulators,
  // the lse and D values, both stages of the K and V tiles, and the S^T and
  // dP^T tiles
  static constexpr int64_t ONCHIP =
      3 * (int64_t)BQB * D + 2 * BQB + 4 * (int64_t)BC * D + 2 * (int64_t)BQB * BC;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
};

// dQ kernel: one workgroup per block of NW * 32 queries, one wave per 32
// queries, K and V tiles of BC keys streamed through LDS.  Per key tile the
// wave recomputes S = Q K^T and P = exp(S - lse), forms dP = dO V^T and
// dS = P o (dP - D), and accumulates dQ^T += K^T dS^T; keys past n are
// masked.  Every LDS address is fixed before the loop (as in bwd_dkdv3):
// each lane's byte offsets for the row-wise K and V reads per k-step and
// the transposed K reads per 32-column block and half are computed once,
// the key sub-block and the k-step only add constants, and the step is
// unrolled by two so that the stage is a constant.  Operands are read two
// MFMAs ahead.
template <int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64, (D >= 256 ? 1 : 8 / NW)) void bwd_dq3(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dg,
    float* __restrict__ dQ, int n, int nqb, int total, float c, float scale) {
  using C = DqCfg<D, NW, BC>;
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int TILE_B = C::TILE * 2;
  __shared__ __attribute__((aligned(1024))) char tiles[4 * TILE_B];  // [stage][K | V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / nqb, qblk = tile - head * nqb;
  const size_t hoff = (size_t)head * n * D;
  const bf16 *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff, *dOh = dO + hoff;
  const int q = qblk * C::BQB + wave * 32 + li;

  bf16x8 qreg[NKK], dogreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qreg[kk] = q < n ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)q * D + 16 * kk + 8 * h)
                     : bf16x8{};
    dogreg[kk] = q < n ? *reinterpret_cast<const bf16x8*>(dOh + (size_t)q * D + 16 * kk + 8 * h)
                       : bf16x8{};
  }
  const float l2 = q < n ? lse[(size_t)head * n + q] * kLog2e : 0.f;
  const float dq_d = q < n ? Dg[(size_t)head * n + q] : 0.f;
  f32x16 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};

  uint32_t koff[C::INSTS], voff[C::INSTS];
#pragma unroll
  for (int it = 0; it < C::INSTS; ++it) {
    const int p = wave * C::WAVE_CHUNKS + it * 64 + lane;
    koff[it] = tile_copy_src<D, dual_swizzle<D * 2>>(p);
    voff[it] = tile_copy_src<D, chunk_swizzle<D * 2>>(p);
  }
  uint32_t rk[NKK], rv[NKK], tk[NDB][2];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    rk[kk] = (uint32_t)row_chunk_elem<D, dual_swizzle<D * 2>>(li, 2 * kk + h) * 2u;
    rv[kk] = (uint32_t)row_chunk_elem<D, chunk_swizzle<D * 2>>(li, 2 * kk + h) * 2u;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int piece = 0; piece < 2; ++piece)
      tk[db][piece] = (uint32_t)tile_elem<D, dual_swizzle<D * 2>>(
                          tr_read_row(lane, piece), db * 32 + tr_read_col(lane)) * 2u;
  // K and V tiles through buffer resources over the head's n rows: rows
  // past n land as zeros (those keys are masked below).
  const rsrc_t rsK = buffer_rsrc(Kh, (uint32_t)n * (D * 2));
  const rsrc_t rsV = buffer_rsrc(Vh, (uint32_t)n * (D * 2));
  const uint32_t tiles_lds = lds_addr(tiles);
  auto load = [&](int j, int stage) {
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(j * BC) * (D * 2);
    const uint32_t kl = tiles_lds + stage * 2 * TILE_B;
#pragma unroll
    for (int it = 0; it < C::INSTS; ++it) {
      const uint32_t p0 = (uint32_t)(wave * C::WAVE_CHUNKS + it * 64) * 16;
      dma16_buf_at(rsK, koff[it], so, kl + p0);
      dma16_buf_at(rsV, voff[it], so, kl + TILE_B + p0);
    }
  };

  const int nkt = (n + BC - 1) / BC;
  auto step = [&](auto stage_c, int j) {
    constexpr int P = decltype(stage_c)::value;
    if (j + 1 < nkt) load(j + 1, P ^ 1);
    const char* Ks = tiles + P * 2 * TILE_B;
    const char* Vs = Ks + TILE_B;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      // Operand sequence: K and V rows alternating over the k-steps of S^T
      // and dP^T, then the transposed K blocks of dQ^T.
      constexpr int NA = 2 * NKK + 2 * NDB, AH = 2;
      bf16x8 a[NA];
      auto fetch = [&](int t) {
        if (t < 2 * NKK) {
          const int kk = t >> 1;
          const char* base = (t & 1) ? Vs : Ks;
          const uint32_t off = (t & 1) ? rv[kk] : rk[kk];
          a[t] = *reinterpret_cast<const bf16x8*>(base + off + kb * 32 * D * 2);
        } else {
          const int u = t - 2 * NKK, ksp = 2 * kb + u / NDB, db = u % NDB;
          const u32x2 p0 =
              lds_read_tr16(reinterpret_cast<const bf16*>(Ks + tk[db][0] + ksp * 16 * D * 2));
          const u32x2 p1 =
              lds_read_tr16(reinterpret_cast<const bf16*>(Ks + tk[db][1] + ksp * 16 * D * 2));
          a[t] = __builtin_bit_cast(bf16x8, (u32x4{p0[0], p0[1], p1[0], p1[1]}));
        }
      };
      auto use = [&](int t) -> bf16x8 {
        if (t + AH < NA) fetch(t + AH);
        return a[t];
      };
#pragma unroll
      for (int t = 0; t < AH; ++t) fetch(t);
      // the compiler's MFMA/LDS interleaving strategy at d = 256 (2.5 %
      // faster there, the same bits; equal at d = 128)
      if constexpr (D >= 256) __builtin_amdgcn_iglp_opt(0);
      // S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries per wave).
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma_bf16_32x32x16(use(2 * kk), qreg[kk], s);
        dp = mfma_bf16_32x32x16(use(2 * kk + 1), dogreg[kk], dp);
      }
      const int kbase = j * BC + kb * 32;
      // keys past n (zero rows of the tile) get s = -inf, so p = 0; one
      // uniform branch for the block keeps the exponentials in one basic
      // block with the MFMAs around them
      if (kbase + 32 > n) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 8 * (r >> 2) + 4 * h + (r & 3) >= n) s[r] = -INFINITY;
      }
      uint32_t dsk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[r], c, -l2));
        const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], c, -l2));
        dsk[r >> 1] = pack_bf16x2(p0 * (dp[r] - dq_d), p1 * (dp[r + 1] - dq_d));
      }
      // dQ^T += K^T dS^T over these 32 keys.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bs = __builtin_bit_cast(
            bf16x8, (u32x4{dsk[4 * ks], dsk[4 * ks + 1], dsk[4 * ks + 2], dsk[4 * ks + 3]}));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dqt[db] = mfma_bf16_32x32x16(use(2 * NKK + ks * NDB + db), bs, dqt[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's copies, before the barrier
    __syncthreads();
  };

  load(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int j = 0;
  for (; j + 1 < nkt; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    step(std::integral_constant<int, 1>{}, j + 1);
  }
  if (j < nkt) step(std::integral_constant<int, 0>{}, j);

  if constexpr (D >= 256) {
    __syncthreads();  // every wave is done with the K and V tiles
    f32x4* const st = reinterpret_cast<f32x4*>(tiles) + wave * 32 * (D / 4);
    const int q0 = qblk * C::BQB + wave * 32;
    store_rows_lds<D>(dqt, scale, st, dQ + hoff + (size_t)q0 * D, n - q0, lane);
  } else if (q < n) {
    float* dQr = dQ + hoff + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a = {dqt[db][4 * g] * scale, dqt[db][4 * g + 1] * scale, dqt[db][4 * g + 2] * scale,
                   dqt[db][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(dQr + db * 32 + 8 * g + 4 * h) = a;
      }
  }
}

// ---------------------------------------------------------------------------
// Host side.

namespace {

// bwd_dkdv3 with NWKV waves (one wave per 32 keys; per 32 queries S, then
// dP, then dV and dK) and bwd_dq3 with NWQ waves (one per 32 queries) and
// BC-key tiles.  The default is eight waves in both and 64-key tiles.
template <int D, int NWKV = 8, int NWQ = 8, int BC = 64>
hipError_t launch(const void* Q, const void* K, const void* V, const float* O, const void* dO,
                  const float* lse, float* dQ, float* dK, float* dV, int64_t bh, int64_t n,
                  float scale, void* ws, hipStream_t stream) {
  const bf16* q = static_cast<const bf16*>(Q);
  const bf16* k = static_cast<const bf16*>(K);
  const bf16* v = static_cast<const bf16*>(V);
  const bf16* g = static_cast<const bf16*>(dO);
  float* Dbuf = static_cast<float*>(ws);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         ((size_t)bh * n * 4 + 255) / 256 * 256);
  const float c = scale * kLog2e;
  const int64_t rows = bh * n;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_preprocess<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, O, g, Dbuf, rows, lse, lse2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  using Ckv = DkdvCfg<D, NWKV>;
  const int nkb = (int)((n + Ckv::BKV - 1) / Ckv::BKV);
  const int total_kv = (int)(bh * nkb);
  hipLaunchKernelGGL((bwd_dkdv3<D, NWKV>), dim3(total_kv), dim3(NWKV * 64), 0, stream, q, k, v,
                     g, lse2, Dbuf, dK, dV, (int)n, nkb, total_kv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  using Cq = DqCfg<D, NWQ, BC>;
  const int nqb = (int)((n + Cq::BQB - 1) / Cq::BQB);
  const int total_q = (int)(bh * nqb);
  hipLaunchKernelGGL((bwd_dq3<D, NWQ, BC>), dim3(total_q), dim3(NWQ * 64), 0, stream, q, k, v,
                     g, lse, Dbuf, dQ, (int)n, nqb, total_q, c, scale);
  return hipGetLastError();
}

// Compiled tile shapes, per head dimension the default first: keys per
// dK/dV workgroup (k), queries per dQ workgroup (q), keys per dQ tile (c).
// Every shape processes each wave's 32 rows in the same order, so all give
// the same bits.
typedef hipError_t (*BwdLaunch)(const void*, const void*, const void*, const float*,
                                const void*, const float*, float*, float*, float*, int64_t,
                                int64_t, float, void*, hipStream_t);
struct BwdEntry {
  const char* name;
  int d;
  BwdTileInfo info;
  BwdLaunch fn;
};

template <int D, int NWKV, int NWQ, int BC>
BwdEntry bwd_entry(const char* name) {
  return BwdEntry{name, D,
                  BwdTileInfo{32 * NWKV, 32 * NWQ, BC,
                              std::max(DkdvCfg<D, NWKV>::ONCHIP, DqCfg<D, NWQ, BC>::ONCHIP)},
                  &launch<D, NWKV, NWQ, BC>};
}

const BwdEntry* bwd_pick(int64_t d, const char* name) {
  static const BwdEntry table[] = {
      bwd_entry<128, 8, 8, 64>("k256q256c64"), bwd_entry<128, 4, 8, 64>("k128q256c64"),
      bwd_entry<128, 8, 4, 64>("k256q128c64"), bwd_entry<128, 8, 8, 32>("k256q256c32"),
      bwd_entry<64, 8, 8, 64>("k256q256c64"),
      // d = 256: four waves, one per SIMD (a wave's dK^T and dV^T alone
      // take 256 of its 512 registers)
      bwd_entry<256, 4, 4, 64>("k128q128c64"),
  };
  for (const BwdEntry& e : table)
    if (e.d == d && (name == nullptr || std::strcmp(name, e.name) == 0)) return &e;
  return nullptr;
}

}  // namespace

hipError_t launch_bwd_preprocess(const float* O, const void* dO, float* Dout, int64_t rows,
                                 int64_t d, hipStream_t stream) {
  const bf16* g = static_cast<const bf16*>(dO);
  switch (d) {
    case 64:
      hipLaunchKernelGGL(bwd_preprocess<64>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0,
                         stream, O, g, Dout, rows, nullptr, nullptr);
      break;
    case 128:
      hipLaunchKernelGGL(bwd_preprocess<128>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                         stream, O, g, Dout, rows, nullptr, nullptr);
      break;
    case 256:
      hipLaunchKernelGGL(bwd_preprocess<256>, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0,
                         stream, O, g, Dout, rows, nullptr, nullptr);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool bwd_supported(int64_t d) { return d == 64 || d == 128 || d == 256; }

int64_t bwd_onchip_elems(int64_t d) { return bwd_tile_info(d).onchip; }

BwdTileInfo bwd_tile_info(int64_t d, const char* tile) {
  const BwdEntry* e = bwd_pick(d, tile);
  return e ? e->info : BwdTileInfo{0, 0, 0, 0};
}

const char* bwd_tile_names(int64_t d) {
  switch (d) {
    case 128: return "k256q256c64 k128q256c64 k256q128c64 k256q256c32";
    case 64: return "k256q256c64";
    case 256: return "k128q128c64";
    default: return "";
  }
}

size_t bwd_workspace_bytes(int64_t bh, int64_t n, int64_t) {
  return 2 * (((size_t)bh * n * 4 + 255) & ~size_t(255));  // D, then lse log2(e)
}

hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const float* O,
                           const void* dO, const float* lse, float* dQ, float* dK, float* dV,
                           int64_t bh, int64_t n, int64_t d, float scale, void* workspace,
                           const char* tile, hipStream_t stream) {
  const BwdEntry* e = bwd_pick(d, tile);
  if (!e) return hipErrorInvalidValue;
  return e->fn(Q, K, V, O, dO, lse, dQ, dK, dV, bh, n, scale, workspace, stream);
}

}  // namespace at
