// Square-tile forward for the small-cache regime (M < d^2).
//
// Method: page "The I/O Complexity of Attention, or How Optimal is Flash
// Attention?" (exposition), section "Small caches: when storing an
// intermediate matrix helps": with square blocks of side b (two input blocks
// and one output block fit in fast memory) every local product reuses each
// loaded element b times, the exponentiated score matrix is written to slow
// memory, and a second tiled product multiplies it by V; the table under
// "Putting the regimes together" gives the N^2 d / sqrt(M) movement term.
//
// Two kernels, stream ordered:
//  1. sc_scores_exp: one workgroup per (head, query tile I, run of jc key
//     tiles J), b x b tiles.  S^T = K_J Q_I^T is accumulated over d in
//     panels of KS columns (64 at b = 128: whole 128-byte lines of the
//     row-major rows; 32 at b = 64): the K and Q panels go global -> LDS
//     with direct copies into a two-slot ring, the next panel's copies run
//     while the current one is multiplied, and the panel pipeline runs on
//     across tile boundaries.  The epilogue takes each query row's maximum over the tile,
//     m_IJ (base-2 units, c = scale log2 e), writes E = exp2(c S - m_IJ) in
//     bf16, and the tile sum l_IJ of the stored bf16 values.  The page does
//     not say how the exponentials are kept in range; the per-tile shift is
//     the reading used here.
//  2. sc_value_product: one workgroup per (head, query tile I, d tile), b x
//     b.  It first merges its rows' statistics: m = max_J m_IJ,
//     l = sum_J 2^(m_IJ - m) l_IJ (the streaming rescale rule applied across
//     tiles), lse = (m + log2 l) ln 2.  Then for each key tile J it
//     accumulates A_J = V_J^T E_IJ^T over 32-key panels (V and E panels
//     global -> LDS with direct copies; V read transposed, E as stored as
//     the MFMA B operand) and adds f_IJ A_J with f_IJ = 2^(m_IJ - m) / l, a
//     per-lane scalar (one query per lane), in fp32 once per key tile.
//
// E is stored in the score kernel's accumulator order, so both kernels move
// it with 16-byte lane accesses that are contiguous per wave: unit
// (head, I, J, wave w, 32-key block kb, half) holds, for each lane, the 8
// bf16 values of accumulator registers 8 half .. 8 half + 7 of that block,
// i.e. keys kb 32 + 16 half + {0..3, 8..11} + 4 (lane / 32) of query
// I b + 32 w + lane % 32.  That key order inside a 16-key step is the one
// the transposed V reads produce, so the contraction pairs every E value
// with its own V row.
//
// Workspace layout (256-byte aligned pieces): E, bh nt^2 b^2 bf16 in the
// unit order above (tiles past n hold finite values that only reach
// discarded rows or are multiplied by 0), then m_IJ [bh][nt][n] and
// l_IJ [bh][nt][n] fp32 with nt = ceil(n/b): key tile major, so the
// statistics of one key tile for consecutive query rows are contiguous
// (each wave writes, merges and stages them as whole 256-byte rows).
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace at {

namespace {

constexpr int KP = 32;  // value product: keys per panel (one 32-key block of E)

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ScLayout {
  size_t e_off, m_off, l_off, total;
  int64_t nt;
};

ScLayout sc_layout(int64_t bh, int64_t n, int64_t b) {
  ScLayout L;
  L.nt = (n + b - 1) / b;
  L.e_off = 0;
  L.m_off = align256((size_t)bh * L.nt * L.nt * b * b * 2);
  L.l_off = L.m_off + align256((size_t)bh * n * L.nt * 4);
  L.total = L.l_off + align256((size_t)bh * n * L.nt * 4);
  return L;
}

// Index of the first 16-byte E unit of (tile (head, I, J), wave, block kb).
template <int B>
__device__ __forceinline__ size_t e_unit(int head, int I, int J, int nt, int wave, int kb) {
  constexpr int NW = B / 32;
  return ((((size_t)head * nt + I) * nt + J) * NW + wave) * (B / 32) * 2 + (size_t)kb * 2;
}

}  // namespace

// Panel pipelines: operand panels are copied global -> LDS ahead of the ones
// being multiplied, into a ring of R slots (DIST = R - 1 panels ahead for the
// scores; two at a time, two ahead, for the value product at R = 4).  The
// on-chip footprint is then b^2 + 2 R_s b KS for the scores (K and Q panels,
// b x KS each) and b bd + R_v (KP bd + b KP) for the value product (V panels
// KP x bd, E panels b x KP).
template <int B>
struct ScScoreCfg {
  // contraction columns per panel: at b = 128 each panel row is one whole
  // 128-byte line of a row-major Q or K row, so no line crosses into the CU
  // twice (two 64-byte strips of a line, a panel apart, would each fetch it)
  static constexpr int KS = B >= 128 ? 64 : 32;
  static constexpr int R = 2;
  static constexpr int DIST = R - 1;
};
template <int B>
struct ScDist {
  static constexpr int R = B >= 128 ? 4 : 2;  // value-product ring slots
};

// ---------------------------------------------------------------------------
// 1. Scores and exponentials of b x b tiles.

template <int D, int B>
__global__ __launch_bounds__(B * 2) void sc_scores_exp(const bf16* __restrict__ Q,
                                                       const bf16* __restrict__ K,
                                                       u32x4* __restrict__ E,
                                                       float* __restrict__ mst,
                                                       float* __restrict__ lst, int n, int nt,
                                                       int jc, int njc, int total, float c) {
  constexpr int KS = ScScoreCfg<B>::KS;
  constexpr int NW = B / 32, NT = NW * 64;
  constexpr int CPR = KS / 8;       // 16-byte chunks per panel row
  constexpr int PCH = B * CPR;      // chunks per panel
  constexpr int LI = PCH / NT;      // copies per lane per panel and operand
  constexpr int NP = D / KS;        // panels per tile
  constexpr int DIST = ScScoreCfg<B>::DIST, R = ScScoreCfg<B>::R;
  static_assert(PCH % NT == 0, "panel chunks must split evenly over the lanes");
  static_assert(NP % R == 0 && DIST < NP, "ring slots must repeat with every tile");
  __shared__ __attribute__((aligned(16))) bf16 Kp[R][B * KS];
  __shared__ __attribute__((aligned(16))) bf16 Qp[R][B * KS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / (nt * njc);
  const int rem = tile - head * nt * njc;
  const int I = rem / njc, jr = rem - (rem / njc) * njc;
  const int J0 = jr * jc, J1 = min(nt, J0 + jc);
  const int q = I * B + wave * 32 + li;
  const bool qok = q < n;

  // Head-wide buffer resources: rows past n read as zeros (their scores
  // are masked, or belong to query rows that are not stored).  Lane chunk
  // p = (wave LI + it) 64 + lane of a panel is row p / CPR, physical chunk
  // p % CPR, which holds logical chunk phys ^ swizzle(row); its byte offset
  // within a panel is per-lane constant, the panel's own offset is scalar.
  const rsrc_t rq = buffer_rsrc(Q + (size_t)head * n * D, (uint32_t)n * (D * 2));
  const rsrc_t rk = buffer_rsrc(K + (size_t)head * n * D, (uint32_t)n * (D * 2));
  uint32_t voff[LI];
#pragma unroll
  for (int it = 0; it < LI; ++it) {
    const int p = (wave * LI + it) * 64 + lane;
    voff[it] = (uint32_t)((p / CPR) * D * 2 + tile_copy_chunk<KS, chunk_swizzle<KS * 2>>(p) * 16);
  }
  // LDS destinations: this wave's part of slot 0 of each ring (scalar)
  const uint32_t wlds = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (LI * 1024u);
  const uint32_t kl = lds_addr(&Kp[0][0]) + wlds, ql = lds_addr(&Qp[0][0]) + wlds;
  // Copy panel pan of key tile J (and of query tile I) into ring slot `slot`.
  auto issue = [&](int J, int pan, int slot) {
    const uint32_t sk = (uint32_t)(J * B * D + pan * KS) * 2u;
    const uint32_t sq = (uint32_t)(I * B * D + pan * KS) * 2u;
    const uint32_t so = (uint32_t)slot * (B * KS * 2);
#pragma unroll
    for (int it = 0; it < LI; ++it) {
      dma16_buf_at(rk, voff[it], sk, kl + so + it * 1024u);
      dma16_buf_at(rq, voff[it], sq, ql + so + it * 1024u);
    }
  };

#pragma unroll
  for (int s = 0; s < DIST; ++s) issue(J0, s, s);
  for (int J = J0; J < J1; ++J) {
    f32x16 acc[B / 32];
#pragma unroll
    for (int pan = 0; pan < NP; ++pan) {
      // Panel (J, pan) was issued DIST steps ago; the loads issued after it
      // are the copies of the next DIST - 1 panels.  Loads complete in issue
      // order, but a store may complete before an older load, so the count
      // covers loads only: with at most that many operations outstanding,
      // no load older than the last DIST - 1 panels' can be.
      wait_vm<(DIST - 1) * 2 * LI>();
      slot_barrier();  // every lane's part of the panel; the slot read last step is free
      {
        // the panel DIST steps ahead; past the end, the last panel again
        // (every step issues the same number of copies)
        int Jn = J + (pan + DIST) / NP, pn = (pan + DIST) % NP;
        if (Jn >= J1) {
          Jn = J1 - 1;
          pn = NP - 1;
        }
        issue(Jn, pn, (pan + DIST) % R);
      }
      const bf16* Ks = Kp[pan % R];
      const bf16* Qs = Qp[pan % R];
      const int qrow = wave * 32 + li;
#pragma unroll
      for (int kk = 0; kk < KS / 16; ++kk) {
        const bf16x8 bq = *reinterpret_cast<const bf16x8*>(
            Qs + row_chunk_elem<KS, chunk_swizzle<KS * 2>>(qrow, 2 * kk + h));
#pragma unroll
        for (int kb = 0; kb < B / 32; ++kb) {
          const int row = kb * 32 + li;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              Ks + row_chunk_elem<KS, chunk_swizzle<KS * 2>>(row, 2 * kk + h));
          acc[kb] = mfma_bf16_32x32x16(a, bq, (pan == 0 && kk == 0) ? f32x16{} : acc[kb]);
        }
      }
    }
    // Epilogue of tile J: tile maximum, exponentials, tile sum.
    if (J == nt - 1 && (n % B) != 0) {
#pragma unroll
      for (int kb = 0; kb < B / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (J * B + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= n) acc[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < B / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m = mx * c;
    float lsum = 0.f;
    u32x4* Eu = E + e_unit<B>(head, I, J, nt, wave, 0) * 64 + lane;
#pragma unroll
    for (int kb = 0; kb < B / 32; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * half + 2 * i;
          pk[i] = pack_bf16x2(fast_exp2(__builtin_fmaf(acc[kb][r], c, -m)),
                              fast_exp2(__builtin_fmaf(acc[kb][r + 1], c, -m)));
          lsum = add_bf16x2(pk[i], lsum);
        }
        // E is read once, by the value product: stream it past the caches
        __builtin_nontemporal_store(u32x4{pk[0], pk[1], pk[2], pk[3]},
                                    &Eu[(kb * 2 + half) * 64]);
      }
    }
    lsum += __shfl_xor(lsum, 32);
    if (qok && h == 0) {
      const size_t sidx = ((size_t)head * nt + J) * n + q;
      mst[sidx] = m;
      lst[sidx] = lsum;
    }
  }
  wait_vm<0>();  // no copy into LDS may outlive the workgroup
}

// ---------------------------------------------------------------------------
// 2. Statistics merge and second product with per-tile row factors.

template <int D, int B>
__global__ __launch_bounds__(B * 2) void sc_value_product(const bf16* __restrict__ V,
                                                          const u32x4* __restrict__ E,
                                                          const float* __restrict__ mst,
                                                          const float* __restrict__ lst,
                                                          float* __restrict__ O,
                                                          float* __restrict__ lse, int n, int nt,
                                                          int total) {
  constexpr int BD = B < D ? B : D;  // d columns per output tile
  constexpr int NCT = D / BD;
  constexpr int NW = B / 32, NT = NW * 64;
  constexpr int CPR = BD / 8;        // 16-byte chunks per V panel row
  constexpr int PCH = KP * CPR;      // chunks per V panel (KP keys)
  constexpr int LI = PCH / NT;
  constexpr int PPT = B / KP;        // panels per key tile
  constexpr int R = ScDist<B>::R;
  constexpr int OPS = LI + 2 + 1;    // copies per lane per panel: V, E (2 units), m_IJ
  static_assert(PCH % NT == 0, "panel chunks must split evenly over the lanes");
  static_assert(KP == 32 && B / 32 == PPT, "one panel is one 32-key block of the score tile");
  __shared__ __attribute__((aligned(16))) bf16 Vp[R][KP * BD];
  __shared__ __attribute__((aligned(16))) bf16 Ep[R][NW * 2 * 64 * 8];  // [wave][half][lane]
  __shared__ __attribute__((aligned(16))) float Ms[R][NW * 64];        // m_IJ per lane

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / (nt * NCT);
  const int rem = tile - head * nt * NCT;
  const int I = rem / NCT, ct = rem - (rem / NCT) * NCT;
  const int q = I * B + wave * 32 + li;
  const bool qok = q < n;

  // merged statistics of this lane's query row
  // statistics are [head][key tile][row]: a wave's 64 rows of one key tile
  // are 256 contiguous bytes
  const float* mr = mst + (size_t)head * nt * n + (qok ? q : 0);
  const float* lr = lst + (size_t)head * nt * n + (qok ? q : 0);
  float m = -INFINITY;
  for (int t = 0; t < nt; ++t) m = fmaxf(m, mr[(size_t)t * n]);
  float l = 0.f;
  for (int t = 0; t < nt; ++t) l += fast_exp2(mr[(size_t)t * n] - m) * lr[(size_t)t * n];
  const float inv = 1.0f / l;
  if (ct == 0 && lse != nullptr && qok && h == 0)
    lse[(size_t)head * n + q] = (m + __log2f(l)) * kLn2;

  // Buffer resources: V of this head (keys past n read as zeros, where E
  // is 0 too), the E units of query tile I ((J, wave, kb, half) order, 1 KiB
  // each) and the statistics of this head.  Per-lane byte offsets are
  // constant; the panel's own offset is scalar.
  const rsrc_t rv = buffer_rsrc(V + (size_t)head * n * D, (uint32_t)n * (D * 2));
  const rsrc_t re = buffer_rsrc(E + e_unit<B>(head, I, 0, nt, 0, 0) * 64,
                                (uint32_t)nt * (NW * PPT * 2 * 1024));
  const rsrc_t rm = buffer_rsrc(mst + (size_t)head * nt * n, (uint32_t)(nt * n) * 4u);
  uint32_t voff[LI];
#pragma unroll
  for (int it = 0; it < LI; ++it) {
    const int p = (wave * LI + it) * 64 + lane;
    voff[it] = (uint32_t)((p / CPR) * D * 2 + ct * BD * 2 +
                          tile_copy_chunk<BD, vtr_swizzle<BD * 2>>(p) * 16);
  }
  const uint32_t eoff = (uint32_t)((wave * PPT * 2) * 1024 + lane * 16);
  // LDS destinations: this wave's part of slot 0 of each ring (scalar)
  const uint32_t wu = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
  const uint32_t vl = lds_addr(&Vp[0][0]) + wu * (LI * 1024u);
  const uint32_t el = lds_addr(&Ep[0][0]) + wu * 2048u;
  const uint32_t ml = lds_addr(&Ms[0][0]) + wu * 256u;
  const uint32_t moff = (uint32_t)(qok ? q : 0) * 4u;
  const int T = nt * PPT;
  // Copy panel t's V, this wave's two E units and each lane's m_IJ into
  // slot t % R.  Panels past the end copy the last one again (same number
  // of copies every step).
  auto issue = [&](int t) {
    t = min(t, T - 1);
    const int J = t / PPT, kb = t - (t / PPT) * PPT, slot = t % R;
    const uint32_t sv = (uint32_t)(J * B + kb * KP) * (D * 2);
#pragma unroll
    for (int it = 0; it < LI; ++it)
      dma16_buf_at(rv, voff[it], sv, vl + slot * (KP * BD * 2) + it * 1024u);
    // E is read once: non-temporal, so V stays cached for the other tiles
    const uint32_t se = (uint32_t)(J * NW * PPT * 2 + kb * 2) * 1024u;
    dma16_buf_nt_at(re, eoff, se, el + slot * (NW * 2 * 1024));
    dma16_buf_nt_at(re, eoff + 1024u, se, el + slot * (NW * 2 * 1024) + 1024u);
    dma4_buf_at(rm, moff, (uint32_t)(J * n) * 4u, ml + slot * (NW * 64 * 4));
  };

  f32x16 out[BD / 32];
#pragma unroll
  for (int db = 0; db < BD / 32; ++db) out[db] = f32x16{};

  // transposed V reads: lane group G = lane / 16 covers d rows 16 (G & 1)
  // .. +15 of a 32-row block and key half hh = G / 2; source lane sl points
  // at key K0 + sl / 4, d D0 + 4 (sl % 4).  The swizzle depends only on the
  // low row bits, which the lane fixes, so each lane's byte offset of a
  // 32-column block is computed once; the 16-key half, the 8-row piece and
  // the ring slot add constants.
  const int G = lane >> 4, sl = lane & 15, hh = G >> 1;
  uint32_t vt_off[BD / 32];
#pragma unroll
  for (int db = 0; db < BD / 32; ++db) {
    const int row0 = 4 * hh + (sl >> 2);
    const int d0 = db * 32 + 16 * (G & 1) + 4 * (sl & 3);
    vt_off[db] =
        (uint32_t)(row0 * BD + ((d0 >> 3) ^ vtr_swizzle<BD * 2>(row0)) * 8 + (d0 & 7)) * 2u;
  }
  const uint32_t e_off = (uint32_t)(((wave * 2) * 64 + lane) * 8) * 2u;

  // PPS panels per barrier: two with a four-slot ring (half the barriers;
  // the next two panels' copies in flight while two are multiplied).
  constexpr int PPS = R >= 4 ? 2 : 1;
  constexpr int AHEAD = R - PPS;  // panels issued ahead of the ones in use
  static_assert(PPT % PPS == 0, "barrier groups must not straddle key tiles");

  // Key tile J: A_J = V_J^T E_IJ^T over its PPT panels, then out += f_IJ A_J.
  // E enters the MFMA as stored (bf16); the row factor is applied in fp32
  // once per tile.  P = (J PPT) % R is the ring slot of the tile's first
  // panel, a constant in each instance.
  auto key_tile = [&](auto phase_c, int J) {
    constexpr int P = decltype(phase_c)::value;
    f32x16 acc[BD / 32];
    float f = 0.f;
#pragma unroll
    for (int kb = 0; kb < PPT; ++kb) {
      const int t = J * PPT + kb;
      const int slot_rt = (P + kb) % R;  // constant after unrolling
      if (kb % PPS == 0) {
        // panels t .. t + PPS - 1 are complete once at most the later
        // AHEAD - PPS panels' copies are outstanding (loads complete in
        // issue order; the only store before this point is older)
        wait_vm<(AHEAD - PPS) * OPS>();
        slot_barrier();  // every lane's part of them; the previous PPS slots are free
#pragma unroll
        for (int p = 0; p < PPS; ++p) issue(t + AHEAD + p);
      }
      if (kb == 0) f = qok ? fast_exp2(Ms[slot_rt][wave * 64 + lane] - m) * inv : 0.f;  // f_IJ
      const char* Vs = reinterpret_cast<const char*>(Vp[slot_rt]);
      const char* Es = reinterpret_cast<const char*>(Ep[slot_rt]);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pb = *reinterpret_cast<const bf16x8*>(Es + e_off + half * 64 * 8 * 2);
#pragma unroll
        for (int db = 0; db < BD / 32; ++db) {
          u32x2 part[2];
#pragma unroll
          for (int piece = 0; piece < 2; ++piece)
            part[piece] = lds_read_tr16(reinterpret_cast<const bf16*>(
                Vs + vt_off[db] + (16 * half + 8 * piece) * BD * 2));
          const bf16x8 a =
              __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
          acc[db] = mfma_bf16_32x32x16(a, pb, (kb == 0 && half == 0) ? f32x16{} : acc[db]);
        }
      }
    }
#pragma unroll
    for (int db = 0; db < BD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[db][r] = __builtin_fmaf(f, acc[db][r], out[db][r]);
  };

#pragma unroll
  for (int s = 0; s < AHEAD; ++s) issue(s);
  for (int J = 0; J < nt; ++J) {
    const int P = (J * PPT) % R;
    if (P == 0) {
      key_tile(std::integral_constant<int, 0>{}, J);
    } else if constexpr (R > 1) {
      if (P == 1) {
        key_tile(std::integral_constant<int, 1 % R>{}, J);
      } else if constexpr (R > 2) {
        key_tile(std::integral_constant<int, 2 % R>{}, J);
      }
    }
  }
  wait_vm<0>();  // no copy into LDS may outlive the workgroup

  if (qok) {
    float* Or = O + ((size_t)head * n + q) * D + ct * BD;
#pragma unroll
    for (int db = 0; db < BD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {out[db][4 * g], out[db][4 * g + 1], out[db][4 * g + 2], out[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(Or + db * 32 + 8 * g + 4 * h) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// Host side.

namespace {

// On-chip elements per workgroup, each counted once whatever its width, and
// every pipeline slot counted: the larger of the two products' footprints.
// Scores: the b x b score tile and R_s = 2 slots each of the K and Q panels
// (LDS, b x KS each, KS = 64 at b = 128, 32 at b = 64).  Value product: the b x bd output tile and R_v slots
// each of the V panel (KP x bd) and the E panel (b x KP), both in LDS,
// R_v = 4 for b = 128, 2 for b = 64; the per-row statistics (b values per
// slot) are not counted.
int64_t footprint(int64_t b, int64_t d) {
  const int64_t bd = b < d ? b : d;
  const int64_t ks = b >= 128 ? 64 : 32;  // ScScoreCfg<b>::KS (R_s = 2)
  const int64_t rv = b >= 128 ? 4 : 2;    // ScDist<b>::R
  const int64_t s = b * b + 2 * 2 * b * ks;
  const int64_t v = b * bd + rv * (KP * bd + b * KP);
  return s > v ? s : v;
}

// Key tiles per score workgroup: enough workgroups to fill the chip twice
// over, and otherwise long runs so the panel pipeline is rarely restarted.
int score_run(int64_t bh, int64_t nt) {
  const int64_t tiles = bh * nt * nt;
  int64_t jc = (tiles + 2047) / 2048;
  if (jc < 1) jc = 1;
  if (jc > nt) jc = nt;
  return (int)jc;
}

template <int D, int B>
hipError_t launch(const void* Q, const void* K, const void* V, float* O, float* lse, int64_t bh,
                  int64_t n, float scale, void* ws, hipStream_t stream) {
  const ScLayout L = sc_layout(bh, n, B);
  // the kernels address one head's E tiles and statistics with 32-bit
  // buffer offsets
  if ((uint64_t)L.nt * B * B * 2 >= (uint64_t(1) << 32) ||
      (uint64_t)L.nt * n * 4 >= (uint64_t(1) << 32))
    return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  u32x4* E = reinterpret_cast<u32x4*>(base + L.e_off);
  float* mst = reinterpret_cast<float*>(base + L.m_off);
  float* lst = reinterpret_cast<float*>(base + L.l_off);
  const int nt = (int)L.nt;
  const float c = scale * kLog2e;

  const int jc = score_run(bh, L.nt);
  const int njc = (nt + jc - 1) / jc;
  const int total1 = (int)(bh * L.nt * njc);
  hipLaunchKernelGGL((sc_scores_exp<D, B>), dim3(total1), dim3(B * 2), 0, stream,
                     static_cast<const bf16*>(Q), static_cast<const bf16*>(K), E, mst, lst,
                     (int)n, nt, jc, njc, total1, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BD = B < D ? B : D;
  const int total2 = (int)(bh * L.nt * (D / BD));
  hipLaunchKernelGGL((sc_value_product<D, B>), dim3(total2), dim3(B * 2), 0, stream,
                     static_cast<const bf16*>(V), E, mst, lst, O, lse, (int)n, nt, total2);
  return hipGetLastError();
}

}  // namespace

// d = 64 is not offered: no supported tile has a footprint below d^2 = 4096.
bool smallcache_supported(int64_t d) { return d == 128 || d == 256; }

int64_t smallcache_onchip_elems(int64_t b) { return (b == 64 || b == 128) ? footprint(b, 256) : 0; }

int64_t smallcache_tile_for_budget(int64_t d, int64_t m_elems) {
  for (int64_t b : {128, 64})
    if (footprint(b, d) <= m_elems && footprint(b, d) < d * d) return b;
  return 0;
}

size_t smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b) {
  return sc_layout(bh, n, b).total;
}

hipError_t launch_fwd_smallcache_bf16(const void* Q, const void* K, const void* V, float* O,
                                      float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                      int64_t b, void* workspace, hipStream_t stream) {
  switch (d * 1000 + b) {
    case 128 * 1000 + 64: return launch<128, 64>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
    case 128 * 1000 + 128:
      return launch<128, 128>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
    case 256 * 1000 + 64: return launch<256, 64>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
    case 256 * 1000 + 128:
      return launch<256, 128>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace at
