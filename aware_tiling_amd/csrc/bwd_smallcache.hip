// Square-tile backward for the small-cache regime (M < d^2).
//
// Method: the page "On Fine-Grained I/O Complexity of Attention Backward
// Passes" (explainer), sections "Methodology" (algorithm design) and "Key
// Contributions and Results" (Theorem 1.1, small cache): below M = d^2 the
// blockwise schedule is not optimal, and the page's Algorithm 6 instead
// writes the n x n attention matrices and n x d intermediates to slow memory
// and works on tiles sized to the cache, for Theta((n^2 d + n d^2)/sqrt(M))
// transfers.  The page prints neither the algorithm's steps nor the
// gradient formulas; the formulas are the exact derivatives of
// O = softmax(scale Q K^T) V,
//     P = exp(scale Q K^T - lse),  dV = P^T dO,  dP = dO V^T,
//     D_i = <dO_i, O_i>,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// and the reading here is the plainest tiled schedule of them in which
// every product is a square-tile matrix product whose on-chip footprint
// (accumulators plus staged panels, each element counted once) fits the
// budget M:
//
//  0. D_i = <dO_i, O_i> (the preprocess kernel of the blockwise backward).
//  1. sb_scores_grads: one workgroup per (head, query tile I, key tile J) of
//     b x b.  S = Q_I K_J^T and dP = dO_I V_J^T are accumulated together over
//     d in panels of 16 columns; the epilogue forms P and dS and writes both,
//     transposed (key-major: P^T[j][i], dS^T[j][i]), in bf16 to the
//     workspace.  Padded rows and columns are written as zeros.
//  2. sb_product (dV and dK in one launch): output tile b keys x b dims,
//     dV_J = P^T_J dO and dK_J = scale dS^T_J Q, contracted over all queries
//     in panels of 16; P^T / dS^T panels are read row-wise, dO / Q panels
//     transposed from LDS.
//  3. sb_product (dQ): dQ_I = scale dS_I K with dS_I read transposed from the
//     key-major dS^T.
//
// Every product is computed transposed (C^T = B^T A^T) so that one lane
// owns one output row and stores four consecutive columns at once.
//
// Workspace (256-byte aligned pieces): D [bh][n] fp32, then P^T and dS^T,
// each bh npad^2 bf16 with npad = ceil(n/b) b, stored panel-major:
// [head][key tile][16-query panel][b keys][16 queries].  A b x 16 panel of
// the dV / dK products is then 4 KB of contiguous memory, a 16 x b panel of
// the dQ product b/16 contiguous pieces of 512 bytes, and a b x b tile of
// the scores kernel 2 b^2 contiguous bytes.
#include "device_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace at {

namespace {

constexpr int SKP = 16;  // contraction panel: one MFMA k-step

__host__ __device__ constexpr size_t sb_align(size_t x) { return (x + 255) & ~size_t(255); }

struct SbLayout {
  size_t d_off, p_off, s_off, total;
  int64_t npad, nt;
};

SbLayout sb_layout(int64_t bh, int64_t n, int64_t b) {
  SbLayout L;
  L.nt = (n + b - 1) / b;
  L.npad = L.nt * b;
  L.d_off = 0;
  L.p_off = sb_align((size_t)bh * n * 4);
  const size_t mat = sb_align((size_t)bh * L.npad * L.npad * 2);
  L.s_off = L.p_off + mat;
  L.total = L.s_off + mat;
  return L;
}

// Element offset of (key j, query i) in a panel-major P^T / dS^T matrix.
template <int B>
__device__ __forceinline__ size_t pt_offset(int head, int j, int i, int nt, int npad) {
  return (((size_t)head * nt + j / B) * (size_t)(npad / 16) + (size_t)(i / 16)) * (B * 16) +
         (size_t)(j % B) * 16 + (i % 16);
}

// Transposed operand (32 columns x 16 panel rows, natural k order) from an
// LDS panel of 16 rows x W bf16 whose 16-byte chunks are swizzled with
// vtr_swizzle: lane l receives column col0 + l%32, rows 8 (l/32) .. +7.
template <int W>
__device__ __forceinline__ bf16x8 tr_panel(const bf16* panel, int col0, int lane) {
  const int G = lane >> 4, sl = lane & 15, hh = G >> 1;
  u32x2 part[2];
#pragma unroll
  for (int piece = 0; piece < 2; ++piece) {
    const int row = 8 * hh + 4 * piece + (sl >> 2);
    const int c = col0 + 16 * (G & 1) + 4 * (sl & 3);
    const int phys = (c >> 3) ^ vtr_swizzle<W * 2>(row);
    part[piece] = lds_read_tr16(panel + row * W + phys * 8 + (c & 7));
  }
  return __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
}

// Direct load of one 16-row x W-column panel (row stride `stride` elements,
// rows clamped to rmax) into LDS with vtr_swizzle, by one wave-load of 64
// lanes per 64 chunks: part `part` covers chunks 64 part .. +63.
template <int W>
__device__ __forceinline__ void load_tr_panel(const bf16* src, int64_t stride, int r0, int rmax,
                                              int c0, bf16* dst, int part, int lane) {
  constexpr int CPR = W / 8;
  const int p0 = part * 64;
  const int p = p0 + lane;
  const int row = p / CPR, phys = p % CPR;
  const int logical = phys ^ vtr_swizzle<W * 2>(row);
  const int grow = min(r0 + row, rmax);
  dma16(src + (size_t)grow * stride + c0 + logical * 8, dst + p0 * 8);
}

// ---------------------------------------------------------------------------
// 1. P and dS of one b x b tile.

// S = Q_I K_J^T is accumulated first, over d in panels of 16 columns, then
// dP = dO_I V_J^T: each step copies two panels (Q and K, or dO and V), so the
// ST stages of four panels the footprint counts make R = 2 ST ring slots of
// two.
template <int D, int B, int ST>
__global__ __launch_bounds__(B * 4) void sb_scores_grads(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dv,
    bf16* __restrict__ Pt, bf16* __restrict__ dSt, int n, int nt, int npad, int total, float c) {
  constexpr int NW = B / 16;
  constexpr int RB = B / 32;  // 32-row query blocks (and wave-loads per tensor panel)
  constexpr int CB = B / 64;  // 32-key blocks per wave
  constexpr int PANEL = B * SKP;
  constexpr int R = 2 * ST;
  static_assert(NW == 2 * RB, "one wave-load per wave covers the step's two panels");
  __shared__ __attribute__((aligned(16))) bf16 sm[R][2][PANEL];  // (Q or dO), (K or V)
  __shared__ __attribute__((aligned(16))) float rowstat[2][B];     // lse, D of the query rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / (nt * nt);
  const int rem = tile - head * nt * nt;
  // b = 128: grouped order, consecutive tiles run over a group of 8 key
  // tiles for each query tile in turn, so the workgroups resident on one
  // XCD at a time read about 8 + 8 row panels of each tensor, which stay in
  // its L2 (in key-major order they read every query tile's panels at once
  // and the streaming P^T / dS^T writes evict them: 6x the HBM reads at
  // d = 256).  b = 64: key-major order, neighbours share the key tile (the
  // grouped order reads more there, with four times the resident tiles).
  int J, I;
  if constexpr (B >= 128) {
    constexpr int GROUP = 8;
    const int g0 = (rem / (GROUP * nt)) * GROUP;
    const int gsize = min(nt - g0, GROUP);
    const int local = rem - g0 * nt;
    J = g0 + local % gsize;
    I = local / gsize;
  } else {
    J = rem / nt;
    I = rem - J * nt;
  }
  const size_t hoff = (size_t)head * n * D;
  const int ib = wave % RB, jh = wave / RB;
  constexpr int NP = D / SKP;
  constexpr int T = 2 * NP;  // steps: NP for S, then NP for dP

  // step t's two panels into slot t % R (steps past the end copy the last
  // one again, so every step issues one copy per lane)
  const int side = wave / RB, part = wave - side * RB;  // side 0: query rows, 1: key rows
  auto issue = [&](int t) {
    t = min(t, T - 1);
    const bool second = t >= NP;
    const int kp = second ? t - NP : t;
    const int p0 = part * 64, p = p0 + lane;
    const int row = p >> 1, hf = p & 1;
    const int grow = min((side == 0 ? I * B : J * B) + row, n - 1);
    const bf16* src = side == 0 ? (second ? dO : Q) : (second ? V : K);
    dma16(src + hoff + (size_t)grow * D + kp * SKP + hf * 8, &sm[t % R][side][p0 * 8]);
  };

  f32x16 s[CB], dp[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) s[cb] = dp[cb] = f32x16{};

  // the query rows' lse and D go to LDS ahead of the panels (the first
  // step's wait covers them): waves 0 .. 2 B / 64 - 1 copy 64 values each
  if (wave < 2 * B / 64) {
    const int which = wave / (B / 64), r0 = (wave % (B / 64)) * 64;
    const int i = min(I * B + r0 + lane, n - 1);
    dma4((which == 0 ? lse : Dv) + (size_t)head * n + i, &rowstat[which][r0]);
  }
  auto compute = [&](int t) {
    const bf16* qs = sm[t % R][0];
    const bf16* ks = sm[t % R][1];
    const int qrow = ib * 32 + li;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&qs[qrow * SKP + h * 8]);
    if (t < NP) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int krow = jh * (B / 2) + cb * 32 + li;
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&ks[krow * SKP + h * 8]);
        s[cb] = mfma_bf16_32x32x16(a, bk, s[cb]);
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int krow = jh * (B / 2) + cb * 32 + li;
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&ks[krow * SKP + h * 8]);
        dp[cb] = mfma_bf16_32x32x16(a, bv, dp[cb]);
      }
    }
  };
  // PPS steps per barrier (two when the ring has four slots: half the
  // barriers, two steps in flight while two are used)
  constexpr int PPS = R >= 4 ? 2 : 1;
  constexpr int AHEAD = R - PPS;  // steps issued ahead of the ones being used
  static_assert(T % PPS == 0, "whole barrier groups");
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) issue(i);
  for (int t = 0; t < T; t += PPS) {
    wait_vm<AHEAD - PPS>();  // steps t .. t+PPS-1 are done; later ones may be in flight
    slot_barrier();               // every lane's copies; the slots of steps t-PPS.. are free
#pragma unroll
    for (int p = 0; p < PPS; ++p) issue(t + AHEAD + p);
#pragma unroll
    for (int p = 0; p < PPS; ++p) compute(t + p);
  }
  wait_vm<0>();  // no copy into LDS may outlive the workgroup

  // Epilogue.  Accumulator register r of a lane holds query row
  // i0 + 8 (r/4) + 4 h + r%4 and key column j of the lane.  P and dS are
  // packed to bf16 in registers; when the panel slots (free now) hold a
  // b x b tile, each tile goes through them so that the P^T / dS^T rows
  // leave as whole 16-byte lane stores, four 2b-byte rows per wave store,
  // instead of 8-byte pieces of 32 rows (the footprint does not grow); else
  // (b = 128 with one stage) the pieces are stored directly.
  const int i0 = I * B + ib * 32;
  uint32_t pp[CB][4][2], pd[CB][4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    // rows i0 + 8 g + 4 h + e of this lane's accumulator registers 4 g + e
    const int ir = ib * 32 + 8 * g + 4 * h;  // row within the tile
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(&rowstat[0][ir]) * kLog2e;
    const f32x4 dd = *reinterpret_cast<const f32x4*>(&rowstat[1][ir]);
    const int i = i0 + 8 * g + 4 * h;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int j = J * B + jh * (B / 2) + cb * 32 + li;
      float p[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const bool ok = j < n && i + e < n;
        p[e] = ok ? fast_exp2(__builtin_fmaf(s[cb][r], c, -l2[e])) : 0.f;
        ds[e] = p[e] * (dp[cb][r] - dd[e]);
      }
      pp[cb][g][0] = pack_bf16x2(p[0], p[1]);
      pp[cb][g][1] = pack_bf16x2(p[2], p[3]);
      pd[cb][g][0] = pack_bf16x2(ds[0], ds[1]);
      pd[cb][g][1] = pack_bf16x2(ds[2], ds[3]);
    }
  }
  if constexpr (sizeof(sm) < (size_t)B * B * 2) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = J * B + jh * (B / 2) + cb * 32 + li;
        const size_t off = pt_offset<B>(head, j, i0 + 8 * g + 4 * h, nt, npad);
        *reinterpret_cast<u32x2*>(Pt + off) = u32x2{pp[cb][g][0], pp[cb][g][1]};
        *reinterpret_cast<u32x2*>(dSt + off) = u32x2{pd[cb][g][0], pd[cb][g][1]};
      }
    return;
  }
  // the b x b tile as [key row][query], 16-byte chunks swizzled by row
  bf16* tileb = &sm[0][0][0];
  constexpr int CPT = B / 8;  // 16-byte chunks per tile row
  auto to_global = [&](const uint32_t (&v)[CB][4][2], bf16* dst) {
    slot_barrier();  // the slots (or the previous tile) are no longer read
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = jh * (B / 2) + cb * 32 + li;  // key within the tile
        const int col = ib * 32 + 8 * g + 4 * h;      // query within the tile
        const int phys = (col >> 3) ^ chunk_swizzle<B * 2>(row);
        *reinterpret_cast<u32x2*>(tileb + row * B + phys * 8 + (col & 7)) =
            u32x2{v[cb][g][0], v[cb][g][1]};
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this lane's tile writes are done
    slot_barrier();
    // the tile is one contiguous region [16-query panel q][key r][16
    // queries]: 16-byte chunk x holds panel q = x / 2b, key r, half c
    bf16* region = dst + pt_offset<B>(head, J * B, I * B, nt, npad);
#pragma unroll
    for (int it = 0; it < B * CPT / (B * 4); ++it) {
      const int x = tid + it * B * 4;
      const int q = x / (2 * B), r = (x % (2 * B)) >> 1, c = x & 1;
      const u32x4 val = *reinterpret_cast<const u32x4*>(
          tileb + r * B + (((2 * q + c) ^ chunk_swizzle<B * 2>(r)) * 8));
      *reinterpret_cast<u32x4*>(region + (size_t)x * 8) = val;
    }
  };
  to_global(pp, Pt);
  to_global(pd, dSt);
}

// ---------------------------------------------------------------------------
// 2/3. Out[r][d] = scale sum_k A(r, k) Bm[k][d] over k < npad, for b x b
// output tiles.  A is P^T or dS^T in the panel-major layout, read with
// r = key (A_TR false: dV, dK) or with r = query (A_TR true: dS^T read as
// dS for dQ); Bm is [n][D] (dO, Q or K).  Up to two jobs share one launch.

struct SbJob {
  const bf16* A;
  const bf16* Bm;
  float* Out;
  float scale;
};

struct SbJobs {
  SbJob job[2];
};

// The product kernels' footprint (b^2 + R 2 b 16) may be as large as the
// scores kernel's (2 b^2 + ST 4 b 16), which decides the tile choice: R =
// b / 32 + 2 ST ring slots of the two panels, filled R - 1 steps ahead.
template <int B, int ST>
struct SbProductRing {
  static constexpr int R = B / 32 + 2 * ST;
};

template <int D, int B, int ST, bool A_TR>
__global__ __launch_bounds__(B * 4) void sb_product(const SbJobs jobs, int n, int nt, int npad,
                                                   int per_job, int total) {
  constexpr int NW = B / 16;
  constexpr int RB = B / 32;   // 32-row output blocks
  constexpr int CB = B / 64;   // 32-column blocks per wave
  constexpr int NDT = D / B;   // column tiles
  constexpr int PANEL = SKP * B;
  constexpr int R = SbProductRing<B, ST>::R, DIST = R - 1;
  static_assert(NW == 2 * RB, "one wave-load per wave covers both panels");
  __shared__ __attribute__((aligned(16))) bf16 sm[R][2][PANEL];  // A panel, Bm panel

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int jb = tile / per_job;
  const int rem = tile - jb * per_job;
  const int head = rem / (nt * NDT);
  const int rem2 = rem - head * nt * NDT;
  const int T = rem2 / NDT, dt = rem2 - T * NDT;
  const SbJob job = jb == 0 ? jobs.job[0] : jobs.job[1];
  const bf16* A = job.A;
  const bf16* Bh = job.Bm + (size_t)head * n * D;
  const int R0 = T * B, C0 = dt * B;
  const int rb = wave % RB, ch = wave / RB;

  const int NP = npad / SKP;
  // panel kp into slot kp % R (panels past the end copy the last one again,
  // so every step issues one copy per lane)
  auto issue = [&](int kp) {
    kp = min(kp, NP - 1);
    const int k0 = kp * SKP, st = kp % R;
    if (wave < RB) {  // A panel: 2B chunks, RB wave-loads
      if constexpr (A_TR) {
        // keys k0 .. k0+15 x queries R0 .. R0+b-1, stored [16][b] with the
        // transposed-read swizzle; chunk p: key row p / (b/8), 8 queries
        constexpr int CPR = B / 8;
        const int p0 = wave * 64, p = p0 + lane;
        const int row = p / CPR, phys = p % CPR;
        const int logical = phys ^ vtr_swizzle<B * 2>(row);
        dma16(A + pt_offset<B>(head, k0 + row, R0 + logical * 8, nt, npad),
                  &sm[st][0][p0 * 8]);
      } else {
        // keys R0 .. R0+b-1 x queries k0 .. k0+15: one contiguous 4 KB panel
        const int p0 = wave * 64, p = p0 + lane;
        dma16(A + pt_offset<B>(head, R0, k0, nt, npad) + (size_t)p * 8, &sm[st][0][p0 * 8]);
      }
    } else {
      load_tr_panel<B>(Bh, D, k0, n - 1, C0, sm[st][1], wave - RB, lane);
    }
  };

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};

  auto compute = [&](int st) {
    // MFMA B operand: A(r = rb*32 + l%32, k = 8h..8h+7)
    bf16x8 bop;
    if constexpr (A_TR)
      bop = tr_panel<B>(sm[st][0], rb * 32, lane);
    else
      bop = *reinterpret_cast<const bf16x8*>(&sm[st][0][(rb * 32 + li) * SKP + h * 8]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const bf16x8 aop = tr_panel<B>(sm[st][1], ch * (B / 2) + cb * 32, lane);
      acc[cb] = mfma_bf16_32x32x16(aop, bop, acc[cb]);
    }
  };

#pragma unroll
  for (int i = 0; i < DIST; ++i) issue(i);
  for (int kp = 0; kp < NP; ++kp) {
    wait_vm<DIST - 1>();  // panel kp is done; the later DIST - 1 may be in flight
    slot_barrier();            // every lane's copy of panel kp; slot (kp - 1) % R is free
    issue(kp + DIST);
    compute(kp % R);
  }
  wait_vm<0>();  // no copy into LDS may outlive the workgroup

  // acc[cb] register r: column C0 + ch B/2 + 32 cb + 8 (r/4) + 4 h + r%4,
  // output row R0 + rb*32 + l%32.
  const int row = R0 + rb * 32 + li;
  if (row < n) {
    float* o = job.Out + ((size_t)head * n + row) * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = C0 + ch * (B / 2) + cb * 32 + 8 * g + 4 * h;
        *reinterpret_cast<f32x4*>(o + col) =
            f32x4{acc[cb][4 * g] * job.scale, acc[cb][4 * g + 1] * job.scale,
                  acc[cb][4 * g + 2] * job.scale, acc[cb][4 * g + 3] * job.scale};
      }
  }
}

template <int D, int B, int ST>
hipError_t launch_sb(const bf16* q, const bf16* k, const bf16* v, const float* O, const bf16* g,
                     const float* lse, float* dQ, float* dK, float* dV, int64_t bh, int64_t n,
                     float scale, void* ws, hipStream_t stream) {
  const SbLayout L = sb_layout(bh, n, B);
  char* base = static_cast<char*>(ws);
  float* Dbuf = reinterpret_cast<float*>(base + L.d_off);
  bf16* Pt = reinterpret_cast<bf16*>(base + L.p_off);
  bf16* dSt = reinterpret_cast<bf16*>(base + L.s_off);
  hipError_t e = launch_bwd_preprocess(O, g, Dbuf, bh * n, D, stream);
  if (e != hipSuccess) return e;
  const int nt = (int)L.nt, npad = (int)L.npad;
  const int total1 = (int)(bh * nt * nt);
  hipLaunchKernelGGL((sb_scores_grads<D, B, ST>), dim3(total1), dim3(B * 4), 0, stream, q, k, v,
                     g, lse, Dbuf, Pt, dSt, (int)n, nt, npad, total1, scale * kLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per_job = (int)(bh * nt * (D / B));
  const SbJobs kv{{SbJob{Pt, g, dV, 1.0f}, SbJob{dSt, q, dK, scale}}};
  hipLaunchKernelGGL((sb_product<D, B, ST, false>), dim3(2 * per_job), dim3(B * 4), 0, stream,
                     kv, (int)n, nt, npad, per_job, 2 * per_job);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const SbJobs qj{{SbJob{dSt, k, dQ, scale}, SbJob{dSt, k, dQ, scale}}};
  hipLaunchKernelGGL((sb_product<D, B, ST, true>), dim3(per_job), dim3(B * 4), 0, stream, qj,
                     (int)n, nt, npad, per_job, per_job);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sb_d(int64_t b, int stages, const bf16* q, const bf16* k, const bf16* v,
                       const float* O, const bf16* g, const float* lse, float* dQ, float* dK,
                       float* dV, int64_t bh, int64_t n, float scale, void* ws,
                       hipStream_t stream) {
  if constexpr (D >= 256) {
    if (b == 128)
      return stages == 2
                 ? launch_sb<D, 128, 2>(q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale, ws, stream)
                 : launch_sb<D, 128, 1>(q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale, ws, stream);
  }
  if (b == 64)
    return stages == 2
               ? launch_sb<D, 64, 2>(q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale, ws, stream)
               : launch_sb<D, 64, 1>(q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale, ws, stream);
  return hipErrorInvalidValue;
}

// Tile choices, largest first: (b, panel stages).
constexpr int kSbChoices[4][2] = {{128, 2}, {128, 1}, {64, 2}, {64, 1}};

}  // namespace

bool bwd_smallcache_supported(int64_t d) { return d == 128 || d == 256; }

int64_t bwd_smallcache_onchip_elems(int64_t b, int64_t stages) {
  // scores/gradients kernel: S and dP accumulators plus four staged panels;
  // product kernels: one b x b accumulator plus two staged panels.
  const int64_t k1 = 2 * b * b + stages * 4 * b * SKP;
  const int64_t k2 = b * b + stages * 2 * b * SKP;
  return k1 > k2 ? k1 : k2;
}

SmallBwdTile bwd_smallcache_tile(int64_t d, int64_t m_elems) {
  if (!bwd_smallcache_supported(d) || m_elems >= d * d) return SmallBwdTile{0, 0};
  for (const auto& ch : kSbChoices) {
    if (ch[0] > d) continue;
    if (bwd_smallcache_onchip_elems(ch[0], ch[1]) <= m_elems) return SmallBwdTile{ch[0], ch[1]};
  }
  return SmallBwdTile{0, 0};
}

size_t bwd_smallcache_workspace_bytes(int64_t bh, int64_t n, int64_t b) {
  return sb_layout(bh, n, b).total;
}

hipError_t launch_bwd_smallcache_bf16(const void* Q, const void* K, const void* V,
                                      const float* O, const void* dO, const float* lse,
                                      float* dQ, float* dK, float* dV, int64_t bh, int64_t n,
                                      int64_t d, float scale, SmallBwdTile t, void* workspace,
                                      hipStream_t stream) {
  const bf16* q = static_cast<const bf16*>(Q);
  const bf16* k = static_cast<const bf16*>(K);
  const bf16* v = static_cast<const bf16*>(V);
  const bf16* g = static_cast<const bf16*>(dO);
  switch (d) {
    case 128:
      return launch_sb_d<128>(t.b, t.stages, q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale,
                              workspace, stream);
    case 256:
      return launch_sb_d<256>(t.b, t.stages, q, k, v, O, g, lse, dQ, dK, dV, bh, n, scale,
                              workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace at
