// Fused streaming attention forward for gfx950 (the large-cache regime).
//
// Method: page "The I/O Complexity of Attention, or How Optimal is Flash
// Attention?" (exposition), sections "Softmax without storing the score
// matrix" (running maximum m, normaliser l and unnormalised output u, updated
// block by block with the rescaling rule) and "Large caches: where
// FlashAttention's I/O comes from" (keep a block of B queries and their
// output state on chip, scan all of K and V once per query block).
//
// Work split: one workgroup per (head, block of B query rows); B = NW * QB *
// 32.  Each wave owns QB*32 query rows and keeps, in registers, its Q rows
// (as MFMA B operands), the transposed output accumulator U^T (d x rows) and
// per row (m, l).  K/V are streamed in tiles of BC keys through
// double-buffered LDS; the tile for step j+1 is fetched into registers while
// step j computes.
//
// Orientation.  The score tile is computed transposed, S^T = K Q^T, so the
// MFMA result puts one query per lane column: a query's scores sit in one
// lane pair (l, l^32), row maxima need only one cross-lane exchange, and the
// rescale factor of a query is a per-lane scalar.  The exponentiated tile
// P^T is converted to bf16 in registers and used directly as the B operand
// of U^T += V^T P^T; the value tile is therefore stored transposed in LDS
// (d rows x BC keys), with the key order permuted (vt_key_pos) to match the
// MFMA accumulator layout, so that each lane's A operand is one 16-byte read.
//
// Exponent base.  Scores are turned into base-2 exponents with one FMA,
// t = s * c - m with c = scale * log2(e), and exponentiated with v_exp_f32.
// m is the running maximum in these units.  To keep the rescale of U off the
// common path, m is only raised when a tile's maximum exceeds it by more
// than kTau (= 8): the stale m keeps every exponential <= 2^8, which fp32
// and bf16 hold exactly as well as values <= 1, and the result is the same
// function because l and U always use the same m.
//
// The row sum l is accumulated from the bf16-rounded P values (the ones the
// MFMA multiplies), so the normalisation matches the weights used.
#include <cstdio>
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace at {

constexpr float kTau = 8.0f;

template <int D, int QB, int NW, int BC>
struct FusedCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * QB * 32;
  static constexpr int KEYS = BC;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per K row
  static constexpr int K_CHUNKS = BC * CPR;          // chunks per K tile
  static constexpr int K_ITERS = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_ITEMS = (BC / 4) * CPR;     // (4 keys x 8 d) blocks per V tile
  static constexpr int V_ITERS = (V_ITEMS + NT - 1) / NT;
  static constexpr int KS = BC * D;                  // bf16 elements per K buffer
  static constexpr int VT = D * BC;                  // bf16 elements per V^T buffer
  static constexpr int LDS_ELEMS = 2 * (KS + VT);
  // Elements held on chip per workgroup: Q block, U block, (m, l) per row,
  // one K tile, one V tile and the score tile (the double buffer is a
  // latency device and is not counted).
  static constexpr int64_t ONCHIP = (int64_t)BR * D * 2 + 2 * BR + 2 * BC * D + (int64_t)BR * BC;
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
};

template <int D, int QB, int NW, int BC>
__global__ __launch_bounds__(NW * 64, 1) void fwd_fused_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    float* __restrict__ O, float* __restrict__ lse, int n, int nqb, int total, float c) {
  using C = FusedCfg<D, QB, NW, BC>;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::LDS_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // Q rows of this wave as B operands: lane holds Q[q][16kk + 8h .. +7].
  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + li;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (q < n)
        qreg[qb][kk] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)q * D + kk * 16 + 8 * h);
      else
        qreg[qb][kk] = bf16x8{};
    }
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
  u32x4 kreg[C::K_ITERS];
  u32x4 vreg[C::V_ITERS][4];

  // Global -> registers for key tile j (rows past n read as zero).
  auto load_tile = [&](int j) {
    const int kbase = j * BC;
#pragma unroll
    for (int it = 0; it < C::K_ITERS; ++it) {
      const int x = tid + it * C::NT;
      const int row = x / C::CPR, cc = x % C::CPR;
      const int key = kbase + row;
      if (x < C::K_CHUNKS && key < n)
        kreg[it] = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + cc * 8);
      else
        kreg[it] = u32x4{};
    }
#pragma unroll
    for (int it = 0; it < C::V_ITERS; ++it) {
      const int x = tid + it * C::NT;
      const int g = x % (BC / 4), cc = x / (BC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kbase + 4 * g + e;
        if (x < C::V_ITEMS && key < n)
          vreg[it][e] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + cc * 8);
        else
          vreg[it][e] = u32x4{};
      }
    }
  };

  // Registers -> LDS buffer `buf`: K row-major with swizzled chunks; V
  // transposed (d rows x BC keys) with permuted key positions.
  auto store_tile = [&](int buf) {
    bf16* Ks = smem + buf * C::KS;
    bf16* Vt = smem + 2 * C::KS + buf * C::VT;
#pragma unroll
    for (int it = 0; it < C::K_ITERS; ++it) {
      const int x = tid + it * C::NT;
      if (x < C::K_CHUNKS) {
        const int row = x / C::CPR, cc = x % C::CPR;
        *reinterpret_cast<u32x4*>(Ks + row * D + ((cc ^ chunk_swizzle<D * 2>(row)) * 8)) =
            kreg[it];
      }
    }
#pragma unroll
    for (int it = 0; it < C::V_ITERS; ++it) {
      const int x = tid + it * C::NT;
      if (x < C::V_ITEMS) {
        const int g = x % (BC / 4), cc = x / (BC / 4);
        const int pos = vt_key_pos(4 * g);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r0 = cc * 8 + 2 * w;
          const int r1 = r0 + 1;
          u32x2 lo = {pair_lo(vreg[it][0][w], vreg[it][1][w]),
                      pair_lo(vreg[it][2][w], vreg[it][3][w])};
          u32x2 hi = {pair_hi(vreg[it][0][w], vreg[it][1][w]),
                      pair_hi(vreg[it][2][w], vreg[it][3][w])};
          *reinterpret_cast<u32x2*>(Vt + r0 * BC +
                                    (((pos >> 3) ^ chunk_swizzle<BC * 2>(r0)) * 8) + (pos & 7)) = lo;
          *reinterpret_cast<u32x2*>(Vt + r1 * BC +
                                    (((pos >> 3) ^ chunk_swizzle<BC * 2>(r1)) * 8) + (pos & 7)) = hi;
        }
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nt) load_tile(j + 1);
    const bf16* Ks = smem + buf * C::KS;
    const bf16* Vt = smem + 2 * C::KS + buf * C::VT;

    // S^T = K_j Q^T: BC x (QB*32), contraction over d.
    f32x16 s[BC / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        const int row = kb * 32 + li;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Ks + row * D + (((2 * kk + h) ^ chunk_swizzle<D * 2>(row)) * 8));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_bf16_32x32x16(a, qreg[qb][kk], s[kb][qb]);
      }
    }

    // Keys past n in the last tile do not exist: their scores are -inf.
    if (j == nt - 1 && (n % BC) != 0) {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BC + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= n) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
          }
        }
    }

    // Online softmax: running maximum, rescale factor, exponentials, sums.
    uint32_t pk[BC / 32][QB][8];
    float alpha[QB];
    bool need_any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mc = mx * c;
      const bool need = mc > m[qb] + kTau;
      const float mn = need ? mc : m[qb];
      alpha[qb] = need ? fast_exp2(m[qb] - mn) : 1.0f;
      need_any |= need;
      m[qb] = mn;
      float lsum = l[qb] * alpha[qb];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][qb][r], c, -mn));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][qb][r + 1], c, -mn));
          const uint32_t pp = pack_bf16x2(p0, p1);
          pk[kb][qb][r >> 1] = pp;
          lsum = add_bf16x2(pp, lsum);
        }
      l[qb] = lsum;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) uacc[db][qb] *= alpha[qb];
    }

    // U^T += V_j^T P^T: contraction over the BC keys in steps of 16.
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
        const int row = db * 32 + li;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Vt + row * BC + (((4 * kb + 2 * half + h) ^ chunk_swizzle<BC * 2>(row)) * 8));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) uacc[db][qb] = mfma_bf16_32x32x16(a, pb[qb], uacc[db][qb]);
      }
    }

    if (j + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: o = u / l, lse = (m + log2 l) ln 2.
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
// LDS buffer.  Each lane holds one element of each MFMA operand, so the
// value tile stays row-major: for the PV step t the lane pair feeds key
// 8(t/4) + 4h + t%4, exactly the key its score register t holds.

template <int D>
struct F32Cfg {
  static constexpr int NW = 4, BC = 32, NT = 256, BR = NW * 32;
  static constexpr int KLD = D + 2;  // padded K row (floats)
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
// Several tile shapes are compiled per head dimension; the first entry of
// each list is the default.  The environment variable ATTN_FWD_TILE
// ("QBxNWxBC", e.g. "1x8x64") selects another compiled shape, for tile
// sweeps; an unknown value falls back to the default.

namespace {

struct FusedEntry {
  int d, qb, nw, bc;
  FusedTileInfo info;
  void (*kernel)(const bf16*, const bf16*, const bf16*, float*, float*, int, int, int, float);
};

template <int D, int QB, int NW, int BC>
FusedEntry entry() {
  using C = FusedCfg<D, QB, NW, BC>;
  return FusedEntry{D, QB, NW, BC, FusedTileInfo{C::BR, C::KEYS, C::ONCHIP},
                    &fwd_fused_bf16_kernel<D, QB, NW, BC>};
}

const FusedEntry* registry(int& count) {
  static const FusedEntry table[] = {
      entry<64, 2, 4, 64>(),  entry<64, 2, 8, 32>(),  entry<64, 2, 4, 32>(),
      entry<128, 1, 8, 64>(), entry<128, 2, 4, 32>(), entry<128, 1, 8, 32>(),
      entry<128, 1, 4, 64>(), entry<256, 1, 4, 32>(),
  };
  count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const FusedEntry* pick(int64_t d) {
  int count = 0;
  const FusedEntry* t = registry(count);
  const FusedEntry* def = nullptr;
  for (int i = 0; i < count; ++i)
    if (t[i].d == d) {
      def = &t[i];
      break;
    }
  if (!def) return nullptr;
  const char* env = getenv("ATTN_FWD_TILE");
  int qb = 0, nw = 0, bc = 0;
  if (env && sscanf(env, "%dx%dx%d", &qb, &nw, &bc) == 3)
    for (int i = 0; i < count; ++i)
      if (t[i].d == d && t[i].qb == qb && t[i].nw == nw && t[i].bc == bc) return &t[i];
  return def;
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

}  // namespace

bool fused_bf16_supported(int64_t d) { return pick(d) != nullptr; }
bool fused_f32_supported(int64_t d) { return d == 64 || d == 128; }

FusedTileInfo fused_bf16_tile_info(int64_t d) {
  const FusedEntry* e = pick(d);
  return e ? e->info : FusedTileInfo{0, 0, 0};
}

FusedTileInfo fused_f32_tile_info(int64_t d) {
  switch (d) {
    case 64: return FusedTileInfo{F32Cfg<64>::BR, F32Cfg<64>::BC, F32Cfg<64>::ONCHIP};
    case 128: return FusedTileInfo{F32Cfg<128>::BR, F32Cfg<128>::BC, F32Cfg<128>::ONCHIP};
    default: return FusedTileInfo{0, 0, 0};
  }
}

hipError_t launch_fwd_fused_bf16(const void* Q, const void* K, const void* V, float* O,
                                 float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                 hipStream_t stream) {
  const FusedEntry* e = pick(d);
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace at
