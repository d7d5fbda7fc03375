// Fused streaming attention forward for gfx950 (the large-cache regime).
//
// Method: page "The I/O Complexity of Attention, or How Optimal is Flash
// Attention?" (exposition), sections "Softmax without storing the score
// matrix" (running maximum m, normaliser l and unnormalised output u, updated
// block by block with the rescaling rule) and "Large caches: where
// FlashAttention's I/O comes from" (keep a block of B queries and their
// output state on chip, scan all of K and V once per query block).
//
// Work split: one workgroup per (head, block of B query rows).  Each wave
// owns 32 query rows and keeps, in registers, its Q rows (as MFMA B
// operands), the transposed output accumulator U^T (d x rows) and per row
// (m, l).  K/V are streamed in tiles of BC keys through LDS.
//
// Orientation.  The score tile is computed transposed, S^T = K Q^T, so the
// MFMA result puts one query per lane column: a query's scores sit in one
// lane pair (l, l^32), row maxima need only one cross-lane exchange, and the
// rescale factor of a query is a per-lane scalar.  The exponentiated tile
// P^T is converted to bf16 in registers and used directly as the B operand
// of U^T += V^T P^T.
//
// Exponent base.  Scores are turned into base-2 exponents with one FMA,
// t = s * c - m with c = scale * log2(e), and exponentiated with v_exp_f32.
// m is the running maximum in these units.  To keep the rescale of U off the
// common path, m is only raised when a tile's maximum exceeds it by more
// than kTau (= 24): the stale m keeps every exponential <= 2^24, which fp32
// and bf16 hold with the same relative precision as values <= 1 (l and U
// stay below n 2^24 max|v|, far from fp32 overflow), and the result is the
// same function because l and U always use the same m.  A row's maximum
// typically grows by about 1.6 score deviations from its first tile to its
// last, so with kTau = 24 rows of score deviation up to about 15 (base 2)
// never rescale after the first tile; any rescale costs the whole wave.
//
// The row sum l is accumulated from the bf16-rounded P values (the ones the
// MFMA multiplies), so the normalisation matches the weights used.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace at {

constexpr float kTau = 24.0f;
constexpr float kSumLimit = 16777216.0f;  // 2^kTau

template <int V>
struct IntC {
  static constexpr int value = V;
};

// ---------------------------------------------------------------------------
// Direct-load variant for gfx950.  K and V tiles travel global -> LDS with
// global_load_lds_dwordx4 (no staging registers, no vector-ALU work), both
// kept row-major in LDS.  The V^T operand of U^T += V^T P^T is read with the
// LDS transpose read ds_read_b64_tr_b16: the four lanes 4e..4e+3 of a
// 16-lane group point at 4 consecutive d values of key K0+e, so each lane
// receives one d column across 4 consecutive keys; two reads give the 8
// k-slots, and K0 of each read follows the key order of the score
// accumulator, so P^T still feeds the MFMA straight from registers.
//
// The schedule is software-pipelined within each wave:
//
//   step j:  issue global -> LDS: K tile j+2, V tile j+1
//            S_{j+1} = K_{j+1} Q^T        (MFMA, LDS K buffer (j+1)%2)
//            softmax(S_j) -> P_j          (VALU)
//            U^T += V_j^T P_j^T           (MFMA, LDS V buffer j%2)
//            wait for this step's copies; barrier
//
// so S_{j+1} runs on the matrix cores while the softmax of S_j runs on the
// vector ALUs.  K runs two tiles ahead of V, so two buffers of each still
// need only one barrier per step: the K buffer written in step j held K_j,
// last read in step j-1, and the V buffer written held V_{j-1}, also last
// read in step j-1.  Steps are unrolled in pairs so every LDS offset is a
// compile-time constant; only the last tile takes the key mask.  Copies go
// through a buffer resource whose range ends at the head's last key, so rows
// past n land as zeros (those keys are masked in the last tile) and no load
// leaves the tensor.

// Arguments of the direct-load forward body.  Queries [bh, nq, d], keys and
// values [bh, nk, d]; outputs [splits, bh, nq, d] and [splits, bh, nq].
struct DirectArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  float* O;
  float* lse;
  int nq, nk, nqb, total, bh, kchunk;
  float c;
  // Tile lists (block-sparse form only): row (mask head, query block) holds
  // counts[row] ascending key-tile indices at tiles + row * tile_cap.
  const int* tiles = nullptr;
  const int* counts = nullptr;
  int tile_cap = 0, mask_heads = 1;
};

// Tags for the K tile (row-wise reads, chunk_swizzle) and the V tile
// (transposed reads, vtr_swizzle), so a loader can pick the matching
// offsets.
template <int ROW_BYTES>
struct KTileSwizzle {
  static constexpr bool is_v = false;
  __device__ int operator()(int row) const { return chunk_swizzle<ROW_BYTES>(row); }
};
template <int ROW_BYTES>
struct VTileSwizzle {
  static constexpr bool is_v = true;
  __device__ int operator()(int row) const { return vtr_swizzle<ROW_BYTES>(row); }
};

template <int D, int NW, int BC>
struct DirectCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;
  static constexpr int KEYS = BC;
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int CHUNKS = BC * CPR;          // per tile, per tensor
  static constexpr int WAVE_CHUNKS = CHUNKS / NW;  // per wave, per tensor
  static constexpr int INSTS = WAVE_CHUNKS / 64;   // load instructions per wave per tensor
  static constexpr int TILE = BC * D;              // bf16 elements per tile
  static constexpr int LDS_ELEMS = 4 * TILE;       // K[2], V[2]
  // on-chip elements of one workgroup, each counted once whatever its width
  // and every pipeline slot counted: Q and U blocks, (m, l), both slots of
  // the K and V rings, the score tiles of the current and the next key tile
  static constexpr int64_t ONCHIP =
      (int64_t)BR * D * 2 + 2 * BR + 4 * BC * D + 2 * (int64_t)BR * BC;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
};

// With SKIP a wave whose 32 query rows all lie past nq still loads its share
// of every tile but does no arithmetic; short query blocks (decoding) then
// cost little beyond the key/value stream.
// With LIST the workgroup visits only the key tiles of its tile list, in
// ascending order; a workgroup with an empty list writes O = 0 and
// lse = -inf (no kept key, no softmax).
template <int D, int NW, int BC, bool SKIP = false, bool LIST = false>
__device__ __forceinline__ void direct_body(const DirectArgs& A) {
  using C = DirectCfg<D, NW, BC>;
  // Row maximum only when a tile's sum shows it moved (one wave per SIMD at
  // d = 256, where the maximum's vector instructions are not hidden by a
  // second wave's matrix work; with two waves per SIMD the test before the
  // value product delays it more than the maximum costs).
  constexpr bool LAZY = D >= 256;
  const float c = A.c;
  __shared__ __attribute__((aligned(1024))) bf16 smem[C::LDS_ELEMS];
  bf16* const Kb = smem;                // [2][TILE]
  bf16* const Vb = smem + 2 * C::TILE;  // [2][TILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int li = lane & 31;

  // Workgroup -> (key split, head, query block); keys of this workgroup are
  // [kbeg, kend), addressed relative to kbeg below (n counts them).
  const int tile = xcd_remap(blockIdx.x, A.total);
  const int per_split = A.bh * A.nqb;
  const int split = tile / per_split;
  const int rem = tile - split * per_split;
  const int head = rem / A.nqb;
  const int qblk = rem - head * A.nqb;
  const int nq = A.nq;
  const int kbeg = split * A.kchunk;
  const int n = min(A.nk, kbeg + A.kchunk) - kbeg;
  const bf16* Qh = A.Q + (size_t)head * nq * D;
  const bf16* Kh = A.K + ((size_t)head * A.nk + kbeg) * D;
  const bf16* Vh = A.V + ((size_t)head * A.nk + kbeg) * D;
  float* const Oh = A.O + ((size_t)split * A.bh + head) * nq * D;
  float* const lseh = A.lse ? A.lse + ((size_t)split * A.bh + head) * nq : nullptr;
  const int q = qblk * C::BR + wave * 32 + li;
  const bool active = !SKIP || qblk * C::BR + wave * 32 < nq;  // wave-uniform

  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qreg[kk] = q < nq ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)q * D + kk * 16 + 8 * h)
                      : bf16x8{};

  f32x16 uacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) uacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const int* tlist = nullptr;
  int nt = (n + BC - 1) / BC;
  if constexpr (LIST) {
    const int row = (A.mask_heads == 1 ? 0 : head) * A.nqb + qblk;
    tlist = A.tiles + (size_t)row * A.tile_cap;
    nt = A.counts[row] * (64 / BC);  // listed tiles are 64 keys: 64 / BC tiles of BC each
    if (nt == 0) {
      if (q < nq) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(Oh + (size_t)q * D + db * 32 + 8 * g + 4 * h) =
                f32x4{0.f, 0.f, 0.f, 0.f};
        if (h == 0 && lseh != nullptr) lseh[q] = -INFINITY;
      }
      return;
    }
  }
  // first key of the t-th tile visited
  auto kbase_of = [&](int t) -> int {
    if constexpr (LIST) {
      constexpr int SUB = 64 / BC;  // BC-key tiles per listed 64-key tile
      // uniform: keeps the base scalar
      return __builtin_amdgcn_readfirstlane(tlist[t / SUB]) * 64 + (t % SUB) * BC;
    } else {
      return t * BC;
    }
  };
  // The second half of the last listed tile can lie wholly past n: dropping
  // it leaves the last tile visited as the only partial one.
  if constexpr (LIST && BC < 64)
    if (kbase_of(nt - 1) >= n) --nt;

  // Issue the copies of tile t of K or V into the LDS tile `dst`.  Lane
  // chunk p of this wave is LDS chunk (row, phys); it fetches logical chunk
  // phys ^ swizzle(row) of that row, at a per-lane byte offset computed once.
  // One buffer resource spans this workgroup's keys of the head and the tile
  // start goes in the scalar offset, so a tile costs no address arithmetic;
  // rows of a partial last tile past n fail the resource's range check and
  // land as zeros (their scores are masked, their values weigh 0).  The
  // copies are issued from inline assembly, so the compiler adds no wait for
  // them before the transposed V reads; each step waits for them before its
  // barrier.
  const KTileSwizzle<D * 2> kswz;
  const VTileSwizzle<D * 2> vswz;
  uint32_t koff[C::INSTS], voff[C::INSTS];
#pragma unroll
  for (int it = 0; it < C::INSTS; ++it) {
    const int p = wave * C::WAVE_CHUNKS + it * 64 + lane;
    koff[it] = tile_copy_src<D, chunk_swizzle<D * 2>>(p);
    voff[it] = tile_copy_src<D, vtr_swizzle<D * 2>>(p);
  }
  const rsrc_t rsK = buffer_rsrc(Kh, (uint32_t)n * (D * 2));
  const rsrc_t rsV = buffer_rsrc(Vh, (uint32_t)n * (D * 2));
  auto load_tile = [&](bf16* dst, int t, auto swz) {
    const bool is_v = decltype(swz)::is_v;
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(kbase_of(t)) * (D * 2);
#pragma unroll
    for (int it = 0; it < C::INSTS; ++it)
      dma16_buf(is_v ? rsV : rsK, is_v ? voff[it] : koff[it], so,
                dst + (wave * C::WAVE_CHUNKS + it * 64) * 8);
  };

  auto compute_s = [&](const bf16* Ks, f32x16 (&s)[BC / 32]) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Ks + row_chunk_elem<D, chunk_swizzle<D * 2>>(kb * 32 + li, 2 * kk + h));
        s[kb] = mfma_bf16_32x32x16(a, qreg[kk], s[kb]);
      }
  };
  // scores of keys past n (a partial last tile) to -inf
  auto mask_keys = [&](f32x16 (&s)[BC / 32], bool mask, int kbase) {
    if (mask) {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= n) s[kb][r] = -INFINITY;
    }
  };
  auto softmax_max = [&](f32x16 (&s)[BC / 32], bool mask, int kbase) {
    mask_keys(s, mask, kbase);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max_xor32(mx);
    const float mc = mx * c;
    const bool need = mc > m + kTau;
    // rare: some lane's maximum moved; lanes that keep m get alpha = 1
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mn = need ? mc : m;
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) uacc[db] *= alpha;
    }
  };
  // P = exp2(c S - m) as packed bf16 and l plus the tile's sum of P
  auto exps = [&](const f32x16 (&s)[BC / 32], uint32_t (&pk)[BC / 32][8]) -> float {
    float lsum = l;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, -m));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, -m));
        const uint32_t pp = pack_bf16x2(p0, p1);
        pk[kb][r >> 1] = pp;
        lsum = add_bf16x2(pp, lsum);
      }
    return lsum;
  };
  // The tile's exponentials, the maximum taken first (softmax_max) or, with
  // LAZY, only when they show that it moved: every weight stays <= 2^kTau
  // while m holds, so a tile sum above 2^kTau (or inf or NaN, as on the
  // first tile, where m = -inf) is the only case that needs the maximum; the
  // tile is then exponentiated again with the updated m.  Both orders give
  // the same P, l and m.
  auto softmax_exp = [&](f32x16 (&s)[BC / 32], uint32_t (&pk)[BC / 32][8]) {
    float lsum = exps(s, pk);
    if constexpr (LAZY) {
      if (__builtin_amdgcn_ballot_w64(!(lsum - l <= kSumLimit)) != 0) {
        softmax_max(s, false, 0);
        lsum = exps(s, pk);
      }
    }
    l = lsum;
  };
  // U^T += V^T P^T with the V^T operand from transposed LDS reads
  // (tr_read_row / tr_read_col: each lane gets one d column across 4 keys,
  // in the score accumulator's key order).
  auto pv = [&](const bf16* Vs, const uint32_t (&pk)[BC / 32][8]) {
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) {
      const int kb = ks >> 1, half = ks & 1;
      u32x4 t = {pk[kb][4 * half + 0], pk[kb][4 * half + 1], pk[kb][4 * half + 2],
                 pk[kb][4 * half + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, t);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        u32x2 part[2];
#pragma unroll
        for (int piece = 0; piece < 2; ++piece)
          part[piece] = lds_read_tr16(Vs + tile_elem<D, vtr_swizzle<D * 2>>(
                                               kb * 32 + 16 * half + tr_read_row(lane, piece),
                                               db * 32 + tr_read_col(lane)));
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
        uacc[db] = mfma_bf16_32x32x16(a, pb, uacc[db]);
      }
    }
  };

  f32x16 s_cur[BC / 32];
  int j = 0;
  // Prologue: K_0, V_0, K_1 into LDS; S_0.
  load_tile(Kb, 0, kswz);
  load_tile(Vb, 0, vswz);
  if (nt > 1) load_tile(Kb + C::TILE, 1, kswz);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (active) compute_s(Kb, s_cur);
  __syncthreads();  // every wave has read K_0 before step 0 overwrites it

  // The next tiles' copies are issued between the score MFMAs and the
  // softmax, not at the top of the step, so that their data returns while
  // the PV MFMAs run instead of during the burst of K operand reads.
  auto step = [&](auto par, int j) {
    constexpr int P = decltype(par)::value;
    f32x16 s_next[BC / 32];
    if (active) {
      if constexpr (!LAZY) softmax_max(s_cur, false, 0);
      compute_s(Kb + (P ^ 1) * C::TILE, s_next);
      // issue each score MFMA's K read four MFMAs ahead of it
      constexpr int NS = (D / 16) * (BC / 32);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i + 4 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // Consecutive tiles need no test: a tile past the end reads zeros into
    // the free slot.  A tile list cannot be read past its length.
    if (!LIST || j + 2 < nt) load_tile(Kb + P * C::TILE, j + 2, kswz);
    load_tile(Vb + (P ^ 1) * C::TILE, j + 1, vswz);
    if (active) {
      uint32_t pk[BC / 32][8];
      softmax_exp(s_cur, pk);
      pv(Vb + P * C::TILE, pk);
    }
    // this step's copies and LDS reads complete before any wave moves on
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) s_cur[kb] = s_next[kb];
  };
  for (; j + 2 < nt; j += 2) {
    step(IntC<0>{}, j);
    step(IntC<1>{}, j + 1);
  }
  if (j + 1 < nt) {
    step(IntC<0>{}, j);
    ++j;
  }
  if (active) {
    uint32_t pk[BC / 32][8];
    const int kbase = kbase_of(j);  // the last tile, partial if it runs past n
    const bool mask = kbase + BC > n;
    if constexpr (LAZY)
      mask_keys(s_cur, mask, kbase);
    else
      softmax_max(s_cur, mask, kbase);
    softmax_exp(s_cur, pk);
    pv(Vb + (j & 1) * C::TILE, pk);
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  if constexpr (D >= 256) {
    // 1 KB output rows: each wave turns its 32 rows around in its quarter of
    // the (now free) K/V ring, half a row (512 bytes) at a time, so that
    // every store instruction writes two whole half-rows; 16-byte chunks are
    // XOR-swizzled by row (row r's chunk c at c ^ r)
    __syncthreads();  // every wave is done with the K/V ring
    f32x4* const st = reinterpret_cast<f32x4*>(smem) + wave * 32 * 32;
    const int qw = qblk * C::BR + wave * 32;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int db4 = 0; db4 < 4; ++db4)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int db = half * 4 + db4;
          const int cidx = db4 * 8 + 2 * g + h;
          st[li * 32 + (cidx ^ li)] = f32x4{uacc[db][4 * g + 0] * inv, uacc[db][4 * g + 1] * inv,
                                            uacc[db][4 * g + 2] * inv, uacc[db][4 * g + 3] * inv};
        }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = it * 64 + lane, r = idx >> 5, cidx = idx & 31;
        const f32x4 v = st[r * 32 + (cidx ^ r)];
        if (qw + r < nq)
          *reinterpret_cast<f32x4*>(Oh + (size_t)(qw + r) * D + half * 128 + cidx * 4) = v;
      }
    }
    if (q < nq && h == 0 && lseh != nullptr) lseh[q] = (m + __log2f(lt)) * kLn2;
  } else if (q < nq) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {uacc[db][4 * g + 0] * inv, uacc[db][4 * g + 1] * inv,
                   uacc[db][4 * g + 2] * inv, uacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Oh + (size_t)q * D + db * 32 + 8 * g + 4 * h) = v;
      }
    if (h == 0 && lseh != nullptr) lseh[q] = (m + __log2f(lt)) * kLn2;
  }
}

// WPS is the number of waves per SIMD the register budget is sized for.
template <int D, int NW, int BC, int WPS>
__global__ __launch_bounds__(NW * 64, (WPS * 4 / NW > 0 ? WPS * 4 / NW : 1)) void
fwd_fused_bf16_direct_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                             const bf16* __restrict__ V, float* __restrict__ O,
                             float* __restrict__ lse, int n, int nqb, int total, float c) {
  direct_body<D, NW, BC, false, false>(
      DirectArgs{Q, K, V, O, lse, n, n, nqb, total, total / nqb, n, c});
}

// Key-split entry: grid = splits x bh x query blocks; split s covers keys
// [s kchunk, (s+1) kchunk) and writes its own normalised output and lse
// (the partials that the merge kernel combines).
template <int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64, (D >= 256 ? 1 : (NW == 1 ? 2 : 8 / NW))) void fwd_split_bf16_kernel(
    const DirectArgs A) {
  direct_body<D, NW, BC, true, false>(A);
}

// Block-sparse entry: one workgroup per (head, 128-query block), visiting
// the key tiles its tile list names.
template <int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64, (D >= 256 ? 1 : (8 / NW > 0 ? 8 / NW : 1))) void fwd_sparse_bf16_kernel(
    const DirectArgs A) {
  direct_body<D, NW, BC, false, true>(A);
}

// Compacts one row of the block mask (mask head, query block) into the
// ascending list of 64-key tiles it keeps: a kept 128-key block contributes
// its two tiles, less a second tile that starts at or past n.  One wave per
// row; ballots give each lane's position in the list.
__global__ __launch_bounds__(64) void sparse_tile_lists(const uint8_t* __restrict__ mask,
                                                        int* __restrict__ tiles,
                                                        int* __restrict__ counts, int nkb, int n,
                                                        int tile_cap) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const uint8_t* mrow = mask + (size_t)row * nkb;
  int* out = tiles + (size_t)row * tile_cap;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
    const int kb = kb0 + lane;
    const bool first = kb < nkb && mrow[kb] != 0;
    const bool second = first && (2 * kb + 1) * 64 < n;
    const uint64_t bf = __builtin_amdgcn_ballot_w64(first);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(second);
    const int pos = base + __popcll(bf & below) + __popcll(bs & below);
    if (first) out[pos] = 2 * kb;
    if (second) out[pos + 1] = 2 * kb + 1;
    base += __popcll(bf) + __popcll(bs);
  }
  if (lane == 0) counts[row] = base;
}

// Combines the key-split partials of each query row with the rescaling
// rule: lse = log sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.  One
// thread per four output columns; partials are [splits][rows][D] and
// [splits][rows].
template <int D>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(const float* __restrict__ Op,
                                                              const float* __restrict__ lsep,
                                                              float* __restrict__ O,
                                                              float* __restrict__ lse,
                                                              int64_t rows, int splits) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mx = fmaxf(mx, lsep[(int64_t)sp * rows + row]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; ++sp) {
    const float w = expf(lsep[(int64_t)sp * rows + row] - mx);
    const f32x4 o = *reinterpret_cast<const f32x4*>(Op + ((int64_t)sp * rows + row) * D + col);
    acc += w * o;
    wsum += w;
  }
  const float inv = 1.0f / wsum;
  *reinterpret_cast<f32x4*>(O + row * D + col) = acc * inv;
  if (col == 0 && lse != nullptr) lse[row] = mx + logf(wsum);
}

// ---------------------------------------------------------------------------
// Ping-pong variant.  The 8 waves form two groups of four (one wave of each
// group per SIMD) that run one phase apart.  Each tile j has a matrix phase
// X_j (S_{j+1} = K_{j+1} Q^T and U^T += V_j^T P_j^T, operands from LDS) and a
// vector phase Y_j (online softmax of S_{j+1} -> P_{j+1}, including the rare
// rescale of U).  With workgroup barriers between phases,
//     slot 2j:   group 0 runs X_j,      group 1 runs Y_{j-1}
//     slot 2j+1: group 0 runs Y_j,      group 1 runs X_j
// so at any time each SIMD has one wave issuing MFMAs and one issuing the
// softmax arithmetic.  Direct loads of K_{j+2} and V_{j+1} are issued at the
// start of slot 2j into the buffers K_j and V_{j-1} left (both groups
// finished X_{j-1} before slot 2j) and waited for at the end of slot 2j+1.
// A wave issues its matrix phase at priority 1 and its vector phase at 0,
// so when both waves of a SIMD are ready the MFMAs go first.

template <int D, int QB, int BC>
struct PingCfg {
  static constexpr int NW = 8, NT = 512;
  static constexpr int BR = NW * QB * 32;
  static constexpr int KEYS = BC;
  static constexpr int CPR = D / 8;
  static constexpr int CHUNKS = BC * CPR;
  static constexpr int WAVE_CHUNKS = CHUNKS / NW;
  static constexpr int INSTS = WAVE_CHUNKS / 64;
  static constexpr int TILE = BC * D;
  static constexpr int LDS_ELEMS = 4 * TILE;
  // as DirectCfg, with one score tile per wave (no next tile in flight)
  static constexpr int64_t ONCHIP =
      (int64_t)BR * D * 2 + 2 * BR + 4 * BC * D + (int64_t)BR * BC;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
};

template <int D, int QB, int BC>
__global__ __launch_bounds__(512, 1) void fwd_fused_bf16_pingpong_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    float* __restrict__ O, float* __restrict__ lse, int n, int nqb, int total, float c) {
  using C = PingCfg<D, QB, BC>;
  __shared__ __attribute__((aligned(1024))) bf16 smem[C::LDS_ELEMS];
  bf16* const Kb = smem;                // [2][TILE]
  bf16* const Vb = smem + 2 * C::TILE;  // [2][TILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int h = lane >> 5;
  const int li = lane & 31;

  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / nqb;
  const int qblk = tile - head * nqb;
  const size_t hoff = (size_t)head * (size_t)n * D;
  const bf16* Qh = Q + hoff;
  const bf16* Kh = K + hoff;
  const bf16* Vh = V + hoff;
  const int qw0 = qblk * C::BR + wave * (QB * 32);

  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + li;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qreg[qb][kk] = q < n ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)q * D + kk * 16 + 8 * h)
                           : bf16x8{};
  }

  f32x16 uacc[D / 32][QB];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) uacc[db][qb] = f32x16{};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
  }
  const int nt = (n + BC - 1) / BC;

  const KTileSwizzle<D * 2> kswz;
  const VTileSwizzle<D * 2> vswz;
  uint32_t koff[C::INSTS], voff[C::INSTS];
#pragma unroll
  for (int it = 0; it < C::INSTS; ++it) {
    const int p = wave * C::WAVE_CHUNKS + it * 64 + lane;
    koff[it] = tile_copy_src<D, chunk_swizzle<D * 2>>(p);
    voff[it] = tile_copy_src<D, vtr_swizzle<D * 2>>(p);
  }
  // Tile copies through one buffer resource per head (K, V) whose range
  // ends at row n: the tile start is a scalar offset, and rows of a partial
  // last tile past n land as zeros (their scores are masked, their values
  // weigh 0).  Issued from inline assembly; each slot's copies are waited
  // for before the barrier that ends it.
  const rsrc_t rsK = buffer_rsrc(Kh, (uint32_t)n * (D * 2));
  const rsrc_t rsV = buffer_rsrc(Vh, (uint32_t)n * (D * 2));
  auto load_tile = [&](bf16* dst, int t, auto swz) {
    const bool is_v = decltype(swz)::is_v;
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(t * BC) * (D * 2);
#pragma unroll
    for (int it = 0; it < C::INSTS; ++it)
      dma16_buf(is_v ? rsV : rsK, is_v ? voff[it] : koff[it], so,
                dst + (wave * C::WAVE_CHUNKS + it * 64) * 8);
  };

  f32x16 s[BC / 32][QB];
  uint32_t pk[BC / 32][QB][8];

  auto compute_s = [&](const bf16* Ks) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Ks + row_chunk_elem<D, chunk_swizzle<D * 2>>(kb * 32 + li, 2 * kk + h));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_bf16_32x32x16(a, qreg[qb][kk], s[kb][qb]);
      }
  };
  auto pv = [&](const bf16* Vs) {
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) {
      const int kb = ks >> 1, half = ks & 1;
      bf16x8 pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        u32x4 t = {pk[kb][qb][4 * half + 0], pk[kb][qb][4 * half + 1], pk[kb][qb][4 * half + 2],
                   pk[kb][qb][4 * half + 3]};
        pb[qb] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        u32x2 part[2];
#pragma unroll
        for (int piece = 0; piece < 2; ++piece)
          part[piece] = lds_read_tr16(Vs + tile_elem<D, vtr_swizzle<D * 2>>(
                                               kb * 32 + 16 * half + tr_read_row(lane, piece),
                                               db * 32 + tr_read_col(lane)));
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) uacc[db][qb] = mfma_bf16_32x32x16(a, pb[qb], uacc[db][qb]);
      }
    }
  };
  // Online softmax of the score tile in `s` (keys from kbase) into pk.
  auto softmax = [&](bool mask, int kbase) {
    if (mask) {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= n) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
          }
    }
    // P against the current m; the row maximum is taken only when a tile
    // sum above 2^kTau (or inf or NaN: the first tile, where m = -inf)
    // shows that it may have moved, and the tile is then exponentiated
    // again: the same P, l and m as with the maximum taken first
    float lsum[QB];
    auto exps = [&]() {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        lsum[qb] = l[qb];
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(__builtin_fmaf(s[kb][qb][r], c, -m[qb]));
            const float p1 = fast_exp2(__builtin_fmaf(s[kb][qb][r + 1], c, -m[qb]));
            const uint32_t pp = pack_bf16x2(p0, p1);
            pk[kb][qb][r >> 1] = pp;
            lsum[qb] = add_bf16x2(pp, lsum[qb]);
          }
      }
    };
    exps();
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over |= !(lsum[qb] - l[qb] <= kSumLimit);
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      bool need_any = false;
      float mn[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = pair_max_xor32(mx);
        const float mc = mx * c;
        const bool need = mc > m[qb] + kTau;
        mn[qb] = need ? mc : m[qb];
        need_any |= need;
      }
      // lanes that keep m get alpha = 1
      if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float alpha = fast_exp2(m[qb] - mn[qb]);
          m[qb] = mn[qb];
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) uacc[db][qb] *= alpha;
        }
      }
      exps();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] = lsum[qb];
  };
  // Matrix phase X_j and vector phase Y_j.
  auto phase_x = [&](int j) {
    __builtin_amdgcn_s_setprio(1);
    if (j + 1 < nt) compute_s(Kb + ((j + 1) & 1) * C::TILE);
    pv(Vb + (j & 1) * C::TILE);
    __builtin_amdgcn_s_setprio(0);
  };
  auto phase_y = [&](int j) {  // softmax of S_{j+1}
    softmax((j + 2 == nt) && (n % BC) != 0, (j + 1) * BC);
  };

  // Prologue: K_0, V_0, K_1; S_0 and P_0 in every wave.
  load_tile(Kb, 0, kswz);
  load_tile(Vb, 0, vswz);
  if (nt > 1) load_tile(Kb + C::TILE, 1, kswz);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  compute_s(Kb);
  softmax(nt == 1 && (n % BC) != 0, 0);
  __syncthreads();  // every wave has read K_0 before slot 0 overwrites it

  // Both groups run the same phase sequence X_0, Y_0, X_1, Y_1, ...; group 1
  // takes one extra barrier first and group 0 one extra barrier last, so
  // group 1 is always one phase behind.  Loads of step j (K_{j+2}, V_{j+1})
  // belong to slot 2j and their wait to the end of slot 2j+1; the group
  // branches below only place those.
  auto loads = [&](int j) {
    if (j + 2 < nt) load_tile(Kb + (j & 1) * C::TILE, j + 2, kswz);
    if (j + 1 < nt) load_tile(Vb + ((j + 1) & 1) * C::TILE, j + 1, vswz);
  };
  if (grp == 1) {
    loads(0);
    __syncthreads();
  }
  for (int j = 0; j < nt; ++j) {
    if (grp == 0) loads(j);
    phase_x(j);
    if (grp == 1) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (grp == 1) loads(j + 1);
    if (j + 1 < nt) phase_y(j);
    if (grp == 0) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();

  float* Oh = O + hoff;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = 1.0f / lt;
    const int q = qw0 + qb * 32 + li;
    if (q < n) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v = {uacc[db][qb][4 * g + 0] * inv, uacc[db][qb][4 * g + 1] * inv,
                     uacc[db][qb][4 * g + 2] * inv, uacc[db][qb][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(Oh + (size_t)q * D + db * 32 + 8 * g + 4 * h) = v;
        }
      if (h == 0 && lse != nullptr) lse[(size_t)head * n + q] = (m[qb] + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: same schedule with v_mfma_f32_32x32x2_f32 and exact per-tile
// rescaling.  One wave per 32 query rows, 4 waves, 32-key tiles, single
// LDS buffer (one wave per SIMD: at d = 256 the Q rows and U take 256 of a
// lane's 512 registers).  Each lane holds one element of each MFMA operand, so the
// value tile stays row-major: for the PV step t the lane pair feeds key
// 8(t/4) + 4h + t%4, exactly the key its score register t holds.

template <int D>
struct F32Cfg {
  static constexpr int NW = 4, BC = 32, NT = 256, BR = NW * 32;
  static constexpr int KLD = D + 2;  // padded K row (floats)
  // single-buffered: Q and U blocks, (m, l), one K and one V tile, the
  // score tile
  static constexpr int64_t ONCHIP = (int64_t)BR * D * 2 + 2 * BR + 2 * BC * D + (int64_t)BR * BC;
};

template <int D>
__global__ __launch_bounds__(256, 1) void fwd_fused_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ lse, int n, int nqb, int total, float c) {
  using C = F32Cfg<D>;
  __shared__ float Ks[C::BC * C::KLD];
  __shared__ __attribute__((aligned(16))) float Vs[C::BC * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / nqb, qblk = tile - head * nqb;
  const size_t hoff = (size_t)head * (size_t)n * D;
  const float *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff;
  const int q = qblk * C::BR + wave * 32 + li;

  float qreg[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qreg[kk] = q < n ? Qh[(size_t)q * D + 2 * kk + h] : 0.f;

  f32x16 uacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) uacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int nt = (n + C::BC - 1) / C::BC;
  for (int j = 0; j < nt; ++j) {
    const int kbase = j * C::BC;
    // Stage K (padded rows) and V (row-major) for this tile.
    for (int x = tid; x < C::BC * D / 4; x += C::NT) {
      const int row = x / (D / 4), c4 = (x % (D / 4)) * 4;
      const int key = kbase + row;
      f32x4 kv = {}, vv = {};
      if (key < n) {
        kv = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + c4);
        vv = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + c4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[row * C::KLD + c4 + e] = kv[e];
      *reinterpret_cast<f32x4*>(Vs + row * D + c4) = vv;
    }
    __syncthreads();

    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) s = mfma_f32_32x32x2(Ks[li * C::KLD + 2 * kk + h], qreg[kk], s);

    if (j == nt - 1 && (n % C::BC) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + 4 * h + (r & 3) >= n) s[r] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx * c);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(__builtin_fmaf(s[r], c, -mn));
      lsum += s[r];
    }
    l = l * alpha + lsum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) uacc[db] *= alpha;

#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int key = 8 * (t >> 2) + 4 * h + (t & 3);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        uacc[db] = mfma_f32_32x32x2(Vs[key * D + db * 32 + li], s[t], uacc[db]);
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  if (q < n) {
    float* Oh = O + hoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {uacc[db][4 * g + 0] * inv, uacc[db][4 * g + 1] * inv, uacc[db][4 * g + 2] * inv,
                   uacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Oh + (size_t)q * D + db * 32 + 8 * g + 4 * h) = v;
      }
    if (h == 0 && lse != nullptr) lse[(size_t)head * n + q] = (m + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Host launchers.
//
// The registry lists the compiled tile shapes per head dimension; the first
// entry for a head dimension is the one attn_fwd uses.  The others are the
// query-block x key-tile shapes of the d = 128 tile sweep (B_r = 32 x waves
// query rows, B_c keys per tile), reachable only through the explicitly
// named entry point attn_fwd_tile.

namespace {

typedef void (*FusedKernel)(const bf16*, const bf16*, const bf16*, float*, float*, int, int, int,
                            float);

struct FusedEntry {
  const char* name;
  int d, nw;
  FusedTileInfo info;
  FusedKernel kernel;
};

template <int D, int NW, int BC, int WPS = 2>
FusedEntry direct(const char* name) {
  using C = DirectCfg<D, NW, BC>;
  return FusedEntry{name, D, NW, FusedTileInfo{C::BR, C::KEYS, C::ONCHIP},
                    &fwd_fused_bf16_direct_kernel<D, NW, BC, WPS>};
}

template <int D, int QB, int BC>
FusedEntry pingpong(const char* name) {
  using C = PingCfg<D, QB, BC>;
  return FusedEntry{name, D, C::NW, FusedTileInfo{C::BR, C::KEYS, C::ONCHIP},
                    &fwd_fused_bf16_pingpong_kernel<D, QB, BC>};
}

const FusedEntry* registry(int& count) {
  static const FusedEntry table[] = {
      // head dimension 64: two 4-wave groups offset by half a tile
      pingpong<64, 2, 64>("g2x64p"),
      // head dimension 128: 8 waves, 64-key tiles
      direct<128, 8, 64>("d8x64"),
      // d = 128 tile sweep (128-key tiles spill registers at d = 128)
      direct<128, 2, 32>("r64c32"),
      direct<128, 2, 64>("r64c64"),
      direct<128, 4, 32>("r128c32"),
      direct<128, 4, 64, 1>("r128c64"),
      direct<128, 8, 32>("r256c32"),
      direct<128, 8, 64>("r256c64"),
      // head dimension 256: 4 waves (one per SIMD), 32-key tiles
      direct<256, 4, 32, 1>("d4x32b"),
  };
  count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

// The default entry for head dimension d, or, with a name, the entry of
// that name for d; nullptr if there is none.
const FusedEntry* pick(int64_t d, const char* name = nullptr) {
  int count = 0;
  const FusedEntry* t = registry(count);
  for (int i = 0; i < count; ++i)
    if (t[i].d == d && (name == nullptr || std::strcmp(t[i].name, name) == 0)) return &t[i];
  return nullptr;
}

template <int D>
hipError_t launch_f32(const float* Q, const float* K, const float* V, float* O, float* lse,
                      int64_t bh, int64_t n, float c, hipStream_t stream) {
  using C = F32Cfg<D>;
  const int nqb = (int)((n + C::BR - 1) / C::BR);
  const int total = (int)(bh * nqb);
  hipLaunchKernelGGL((fwd_fused_f32_kernel<D>), dim3(total), dim3(C::NT), 0, stream, Q, K, V, O,
                     lse, (int)n, nqb, total, c);
  return hipGetLastError();
}

// Key-split (rectangular / decoding) forward: the direct kernel in its
// SKIP form with one wave and 32-key tiles when a head has at most 32
// queries (decoding: a 32 KB K/V ring, so five workgroups share a CU and
// no wave sits idle), four waves (128-row query blocks) up to 128 queries,
// else eight; at d = 256 always four waves (one per SIMD) and 32-key tiles,
// the shape of the d = 256 fused forward.
typedef void (*SplitKernel)(DirectArgs);

template <int D>
hipError_t launch_split(const void* Q, const void* K, const void* V, float* O, float* lse,
                        int64_t bh, int64_t nq, int64_t nk, float c, int64_t splits,
                        void* workspace, hipStream_t stream) {
  const bool narrow = D >= 256 || nq <= 128;
  const bool single = D <= 128 && nq <= 32;
  const int nw = single ? 1 : narrow ? 4 : 8;
  SplitKernel kern;
  if constexpr (D >= 256)
    kern = &fwd_split_bf16_kernel<D, 4, 32>;
  else
    kern = single   ? &fwd_split_bf16_kernel<D, 1, 32>
           : narrow ? &fwd_split_bf16_kernel<D, 4, 64>
                    : &fwd_split_bf16_kernel<D, 8, 64>;
  const int br = nw * 32;
  const int64_t kchunk = splitk_key_chunk(nk, splits);
  const int64_t eff = (nk + kchunk - 1) / kchunk;
  const int nqb = (int)((nq + br - 1) / br);
  const int total = (int)(eff * bh * nqb);
  float* Op = O;
  float* lsep = lse;
  if (eff > 1) {
    Op = static_cast<float*>(workspace);
    lsep = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    align256_bytes((size_t)(splits * bh * nq * D) * 4));
  }
  const DirectArgs args{static_cast<const bf16*>(Q), static_cast<const bf16*>(K),
                        static_cast<const bf16*>(V), Op, lsep, (int)nq, (int)nk, nqb, total,
                        (int)bh, (int)kchunk, c};
  hipLaunchKernelGGL(kern, dim3(total), dim3(nw * 64), 0, stream, args);
  if (eff > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = bh * nq;
    constexpr int RPB = 256 / (D / 4);
    hipLaunchKernelGGL((fwd_split_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(256), 0, stream, Op, lsep, O, lse, rows, (int)eff);
  }
  return hipGetLastError();
}

}  // namespace

size_t align256_bytes(size_t b) { return (b + 255) / 256 * 256; }

bool splitk_supported(int64_t d) { return d == 64 || d == 128 || d == 256; }

// Automatic chunk count.  The eight-wave form (more than 128 queries per
// head) is bound by the matrix core and one workgroup fills a CU, so one
// round of 256 workgroups is the target (more chunks only add merge
// traffic); the four-wave form serves short query blocks, bound by the K/V
// stream, where two rounds of its two-per-CU workgroups (1024) keep the most
// loads in flight; the one-wave decoding form (at most 32 queries, d <= 128)
// runs five workgroups per CU, and 512 of them (two per CU, the chunks
// twice as long) were the fastest.  Measured on the decode and chunk
// workloads: 2 and 2 chunks.
int64_t splitk_auto_splits(int64_t bh, int64_t nq, int64_t nk, int64_t d) {
  const bool single = d <= 128 && nq <= 32;
  const bool narrow = nq <= 128;
  const int64_t br = single ? 32 : narrow ? 128 : 256;
  const int64_t target = single ? 512 : narrow ? 1024 : 256;
  const int64_t wgs = bh * ((nq + br - 1) / br);
  int64_t s = (target + wgs - 1) / wgs;
  s = std::min<int64_t>(s, (nk + 255) / 256);  // at least 256 keys per chunk
  return std::max<int64_t>(1, std::min<int64_t>(s, 256));
}

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
  return align256_bytes((size_t)(splits * bh * nq * d) * 4) +
         align256_bytes((size_t)(splits * bh * nq) * 4);
}

hipError_t launch_fwd_splitk_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t nq, int64_t nk, int64_t d,
                                  float scale, int64_t splits, void* workspace,
                                  hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (d) {
    case 64: return launch_split<64>(Q, K, V, O, lse, bh, nq, nk, c, splits, workspace, stream);
    case 128: return launch_split<128>(Q, K, V, O, lse, bh, nq, nk, c, splits, workspace, stream);
    case 256: return launch_split<256>(Q, K, V, O, lse, bh, nq, nk, c, splits, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

// Scratch of the allocation-free key-split forward: the per-chunk partial
// O and lse live in this file-scope device array (one copy per GPU the
// library is loaded on, kept until the process ends) instead of a caller's
// workspace.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[kSplitkScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_splitk_noalloc_bf16(const void* Q, const void* K, const void* V, float* O,
                                          float* lse, int64_t bh, int64_t nq, int64_t nk,
                                          int64_t d, float scale, int64_t splits,
                                          hipStream_t stream) {
  void* ws = nullptr;
  if (splitk_workspace_bytes(bh, nq, nk, d, splits) > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_fwd_splitk_bf16(Q, K, V, O, lse, bh, nq, nk, d, scale, splits, ws, stream);
}

size_t sparse_workspace_bytes(int64_t n, int64_t mask_heads) {
  const int64_t nqb = (n + kSparseBlock - 1) / kSparseBlock;
  const int64_t cap = (n + 63) / 64;
  return align256_bytes((size_t)(mask_heads * nqb) * 4) +
         align256_bytes((size_t)(mask_heads * nqb * cap) * 4);
}

hipError_t launch_fwd_sparse_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                  const uint8_t* mask, int64_t mask_heads, void* workspace,
                                  hipStream_t stream) {
  const int nqb = (int)((n + kSparseBlock - 1) / kSparseBlock);
  const int cap = (int)((n + 63) / 64);
  int* counts = static_cast<int*>(workspace);
  int* tiles = reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                      align256_bytes((size_t)(mask_heads * nqb) * 4));
  hipLaunchKernelGGL(sparse_tile_lists, dim3((unsigned)(mask_heads * nqb)), dim3(64), 0, stream,
                     mask, tiles, counts, nqb, (int)n, cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = (int)(bh * nqb);
  DirectArgs args{static_cast<const bf16*>(Q), static_cast<const bf16*>(K),
                  static_cast<const bf16*>(V), O, lse, (int)n, (int)n, nqb, total, (int)bh,
                  (int)n, scale * kLog2e};
  args.tiles = tiles;
  args.counts = counts;
  args.tile_cap = cap;
  args.mask_heads = (int)mask_heads;
  switch (d) {
    case 64:
      hipLaunchKernelGGL((fwd_sparse_bf16_kernel<64, 4, 64>), dim3(total), dim3(256), 0, stream,
                         args);
      break;
    case 128:
      hipLaunchKernelGGL((fwd_sparse_bf16_kernel<128, 4, 64>), dim3(total), dim3(256), 0, stream,
                         args);
      break;
    case 256:  // four waves (one per SIMD), two 32-key tiles per listed tile
      hipLaunchKernelGGL((fwd_sparse_bf16_kernel<256, 4, 32>), dim3(total), dim3(256), 0, stream,
                         args);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool fused_bf16_supported(int64_t d) { return pick(d) != nullptr; }
bool fused_f32_supported(int64_t d) { return d == 64 || d == 128 || d == 256; }

FusedTileInfo fused_bf16_tile_info(int64_t d, const char* tile) {
  const FusedEntry* e = pick(d, tile);
  return e ? e->info : FusedTileInfo{0, 0, 0};
}

const char* fused_bf16_tile_names(int64_t d) {
  // Space-separated names per head dimension, built once (function-local
  // static: thread-safe initialisation).
  struct Names {
    char s[3][160] = {};
    Names() {
      int count = 0;
      const FusedEntry* t = registry(count);
      const int dims[3] = {64, 128, 256};
      for (int k = 0; k < 3; ++k) {
        size_t len = 0;
        for (int i = 0; i < count; ++i) {
          if (t[i].d != dims[k]) continue;
          const size_t w = std::strlen(t[i].name);
          if (len + w + 2 > sizeof(s[k])) break;
          if (len) s[k][len++] = ' ';
          std::memcpy(s[k] + len, t[i].name, w);
          len += w;
        }
      }
    }
  };
  static const Names names;
  return d == 64 ? names.s[0] : d == 128 ? names.s[1] : d == 256 ? names.s[2] : "";
}

FusedTileInfo fused_f32_tile_info(int64_t d) {
  switch (d) {
    case 64: return FusedTileInfo{F32Cfg<64>::BR, F32Cfg<64>::BC, F32Cfg<64>::ONCHIP};
    case 128: return FusedTileInfo{F32Cfg<128>::BR, F32Cfg<128>::BC, F32Cfg<128>::ONCHIP};
    case 256: return FusedTileInfo{F32Cfg<256>::BR, F32Cfg<256>::BC, F32Cfg<256>::ONCHIP};
    default: return FusedTileInfo{0, 0, 0};
  }
}

hipError_t launch_fwd_fused_bf16(const void* Q, const void* K, const void* V, float* O,
                                 float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                 const char* tile, hipStream_t stream) {
  const FusedEntry* e = pick(d, tile);
  if (!e) return hipErrorInvalidValue;
  const int nqb = (int)((n + e->info.block_rows - 1) / e->info.block_rows);
  const int total = (int)(bh * nqb);
  hipLaunchKernelGGL(e->kernel, dim3(total), dim3(e->nw * 64), 0, stream,
                     static_cast<const bf16*>(Q), static_cast<const bf16*>(K),
                     static_cast<const bf16*>(V), O, lse, (int)n, nqb, total, scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd_fused_f32(const float* Q, const float* K, const float* V, float* O,
                                float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (d) {
    case 64: return launch_f32<64>(Q, K, V, O, lse, bh, n, c, stream);
    case 128: return launch_f32<128>(Q, K, V, O, lse, bh, n, c, stream);
    case 256: return launch_f32<256>(Q, K, V, O, lse, bh, n, c, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace at
