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
// Three kernels, stream ordered:
//  1. sc_scores_exp: one workgroup per (head, query tile I, key tile J), b x b.
//     S^T = K_J Q_I^T is accumulated over d in panels of KP = 32 columns
//     staged in LDS.  The epilogue takes each query row's maximum over the
//     tile, m_IJ (base-2 units, c = scale log2 e), writes
//     E = exp2(c S - m_IJ) in bf16 to the workspace, and the tile sum l_IJ of
//     the stored bf16 values.  The page does not say how the exponentials are
//     kept in range; the per-tile shift is the reading used here.
//  2. sc_merge_stats: per query row, m = max_J m_IJ, l = sum_J 2^(m_IJ - m)
//     l_IJ (the streaming rescale rule applied across tiles), then the factor
//     f_IJ = 2^(m_IJ - m) / l overwrites m_IJ, and lse = (m + log2 l) ln 2.
//  3. sc_value_product: one workgroup per (head, query tile I, d tile), b x
//     b.  For each key tile J, A_J = V_J^T E_IJ^T is accumulated over keys in
//     panels of KP (V panel transposed into LDS, E read as MFMA B operand),
//     then O^T += f_IJ * A_J with f a per-lane scalar (one query per lane).
//
// Workspace layout (256-byte aligned pieces): E [bh][n][npad] bf16 with
// npad = ceil(n/b) b (padded keys hold 0), then stats m|f [bh][n][nt] and
// l [bh][n][nt] fp32 with nt = ceil(n/b).
#include "device_common.h"
#include "launch.h"

namespace at {

namespace {

constexpr int KP = 32;  // contraction panel width (elements)

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ScLayout {
  size_t e_off, m_off, l_off, total;
  int64_t npad, nt;
};

ScLayout sc_layout(int64_t bh, int64_t n, int64_t b) {
  ScLayout L;
  L.nt = (n + b - 1) / b;
  L.npad = L.nt * b;
  L.e_off = 0;
  L.m_off = align256((size_t)bh * n * L.npad * 2);
  L.l_off = L.m_off + align256((size_t)bh * n * L.nt * 4);
  L.total = L.l_off + align256((size_t)bh * n * L.nt * 4);
  return L;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. Scores and exponentials of one b x b tile.

template <int D, int B>
__global__ __launch_bounds__(B * 2, 1) void sc_scores_exp(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, bf16* __restrict__ E,
    float* __restrict__ mst, float* __restrict__ lst, int n, int nt, int npad, int total,
    float c) {
  constexpr int NW = B / 32, NT = NW * 64;
  constexpr int CH = KP / 8;                // 16-byte chunks per panel row
  constexpr int PCH = B * CH;               // chunks per panel
  constexpr int ITERS = (PCH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 Qp[2][B * KP];
  __shared__ __attribute__((aligned(16))) bf16 Kp[2][B * KP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / (nt * nt);
  const int rem = tile - head * nt * nt;
  const int I = rem / nt, J = rem - (rem / nt) * nt;
  const size_t hoff = (size_t)head * n * D;
  const bf16* Qh = Q + hoff;
  const bf16* Kh = K + hoff;

  u32x4 qr[ITERS], kr[ITERS];
  auto load = [&](int p) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int x = tid + it * NT;
      const int row = x / CH, cc = x % CH;
      const int q = I * B + row, key = J * B + row;
      const bool ok = x < PCH;
      qr[it] = (ok && q < n) ? *reinterpret_cast<const u32x4*>(Qh + (size_t)q * D + p * KP + cc * 8)
                             : u32x4{};
      kr[it] = (ok && key < n)
                   ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + p * KP + cc * 8)
                   : u32x4{};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int x = tid + it * NT;
      if (x < PCH) {
        const int row = x / CH, cc = x % CH;
        const int off = row * KP + ((cc ^ chunk_swizzle<KP * 2>(row)) * 8);
        *reinterpret_cast<u32x4*>(&Qp[buf][off]) = qr[it];
        *reinterpret_cast<u32x4*>(&Kp[buf][off]) = kr[it];
      }
    }
  };

  f32x16 acc[B / 32];
#pragma unroll
  for (int kb = 0; kb < B / 32; ++kb) acc[kb] = f32x16{};

  constexpr int NP = D / KP;
  load(0);
  store(0);
  __syncthreads();
  for (int p = 0; p < NP; ++p) {
    const int buf = p & 1;
    if (p + 1 < NP) load(p + 1);
#pragma unroll
    for (int kk = 0; kk < KP / 16; ++kk) {
      const int qrow = wave * 32 + li;
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(
          &Qp[buf][qrow * KP + (((2 * kk + h) ^ chunk_swizzle<KP * 2>(qrow)) * 8)]);
#pragma unroll
      for (int kb = 0; kb < B / 32; ++kb) {
        const int krow = kb * 32 + li;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &Kp[buf][krow * KP + (((2 * kk + h) ^ chunk_swizzle<KP * 2>(krow)) * 8)]);
        acc[kb] = mfma_bf16_32x32x16(a, bq, acc[kb]);
      }
    }
    if (p + 1 < NP) store(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: tile maximum, exponentials, tile sum.
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
  const int q = I * B + wave * 32 + li;
  float lsum = 0.f;
  bf16* Er = E + ((size_t)head * n + (q < n ? q : 0)) * npad + (size_t)J * B;
#pragma unroll
  for (int kb = 0; kb < B / 32; ++kb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t p01 = pack_bf16x2(fast_exp2(__builtin_fmaf(acc[kb][4 * g + 0], c, -m)),
                                       fast_exp2(__builtin_fmaf(acc[kb][4 * g + 1], c, -m)));
      const uint32_t p23 = pack_bf16x2(fast_exp2(__builtin_fmaf(acc[kb][4 * g + 2], c, -m)),
                                       fast_exp2(__builtin_fmaf(acc[kb][4 * g + 3], c, -m)));
      lsum = add_bf16x2(p23, add_bf16x2(p01, lsum));
      if (q < n) *reinterpret_cast<u32x2*>(Er + kb * 32 + 8 * g + 4 * h) = u32x2{p01, p23};
    }
  lsum += __shfl_xor(lsum, 32);
  if (q < n && h == 0) {
    const size_t s = ((size_t)head * n + q) * nt + J;
    mst[s] = m;
    lst[s] = lsum;
  }
}

// ---------------------------------------------------------------------------
// 2. Merge the per-tile statistics of each query row.

__global__ __launch_bounds__(256) void sc_merge_stats(float* __restrict__ mst,
                                                      const float* __restrict__ lst,
                                                      float* __restrict__ lse, int64_t rows,
                                                      int nt) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float* mr = mst + r * nt;
  const float* lr = lst + r * nt;
  float m = -INFINITY;
  for (int t = 0; t < nt; ++t) m = fmaxf(m, mr[t]);
  float l = 0.f;
  for (int t = 0; t < nt; ++t) l += fast_exp2(mr[t] - m) * lr[t];
  const float inv = 1.0f / l;
  for (int t = 0; t < nt; ++t) mr[t] = fast_exp2(mr[t] - m) * inv;
  if (lse) lse[r] = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// 3. Second product with per-tile row factors.

template <int D, int B>
__global__ __launch_bounds__(B * 2, 1) void sc_value_product(
    const bf16* __restrict__ V, const bf16* __restrict__ E, const float* __restrict__ fst,
    float* __restrict__ O, int n, int nt, int npad, int total) {
  constexpr int BD = B < D ? B : D;          // d columns per output tile
  constexpr int NCT = D / BD;
  constexpr int NW = B / 32, NT = NW * 64;
  constexpr int ITEMS = (KP / 4) * (BD / 8);  // (4 keys x 8 d) blocks per V panel
  constexpr int ITERS = (ITEMS + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][BD * KP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / (nt * NCT);
  const int rem = tile - head * nt * NCT;
  const int I = rem / NCT, ct = rem - (rem / NCT) * NCT;
  const bf16* Vh = V + (size_t)head * n * D + ct * BD;
  const int q = I * B + wave * 32 + li;
  const bf16* Er = E + ((size_t)head * n + (q < n ? q : 0)) * npad;
  const float* fr = fst + ((size_t)head * n + (q < n ? q : 0)) * nt;

  u32x4 vr[ITERS][4];
  auto load = [&](int kbase) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int x = tid + it * NT;
      const int g = x % (KP / 4), cc = x / (KP / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kbase + 4 * g + e;
        vr[it][e] = (x < ITEMS && key < n)
                        ? *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + cc * 8)
                        : u32x4{};
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int x = tid + it * NT;
      if (x < ITEMS) {
        const int g = x % (KP / 4), cc = x / (KP / 4);
        const int pos = 4 * g;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r0 = cc * 8 + 2 * w, r1 = r0 + 1;
          u32x2 lo = {pair_lo(vr[it][0][w], vr[it][1][w]), pair_lo(vr[it][2][w], vr[it][3][w])};
          u32x2 hi = {pair_hi(vr[it][0][w], vr[it][1][w]), pair_hi(vr[it][2][w], vr[it][3][w])};
          *reinterpret_cast<u32x2*>(
              &Vt[buf][r0 * KP + (((pos >> 3) ^ chunk_swizzle<KP * 2>(r0)) * 8) + (pos & 7)]) = lo;
          *reinterpret_cast<u32x2*>(
              &Vt[buf][r1 * KP + (((pos >> 3) ^ chunk_swizzle<KP * 2>(r1)) * 8) + (pos & 7)]) = hi;
        }
      }
    }
  };

  f32x16 out[BD / 32], acc[BD / 32];
#pragma unroll
  for (int db = 0; db < BD / 32; ++db) out[db] = acc[db] = f32x16{};

  constexpr int PPT = B / KP;  // panels per key tile
  const int np = nt * PPT;
  load(0);
  store(0);
  __syncthreads();
  for (int p = 0; p < np; ++p) {
    const int buf = p & 1;
    if (p + 1 < np) load((p + 1) * KP);
#pragma unroll
    for (int ks = 0; ks < KP / 16; ++ks) {
      const bf16x8 be = q < n ? *reinterpret_cast<const bf16x8*>(Er + p * KP + ks * 16 + 8 * h)
                              : bf16x8{};
#pragma unroll
      for (int db = 0; db < BD / 32; ++db) {
        const int row = db * 32 + li;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &Vt[buf][row * KP + (((2 * ks + h) ^ chunk_swizzle<KP * 2>(row)) * 8)]);
        acc[db] = mfma_bf16_32x32x16(a, be, acc[db]);
      }
    }
    if ((p + 1) % PPT == 0) {
      const float f = q < n ? fr[p / PPT] : 0.f;
#pragma unroll
      for (int db = 0; db < BD / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) out[db][r] = __builtin_fmaf(f, acc[db][r], out[db][r]);
        acc[db] = f32x16{};
      }
    }
    if (p + 1 < np) store(buf ^ 1);
    __syncthreads();
  }

  if (q < n) {
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
// every pipeline stage counted: the larger of the two products' footprints.
// Scores: the b x b score tile and two stages of the Q and K panels (b x KP
// each).  Value product: the b x bd output tile, the b x bd partial for the
// current key tile, the E panel in registers (b x KP) and two stages of the
// V panel (KP x bd).
int64_t footprint(int64_t b, int64_t d) {
  const int64_t bd = b < d ? b : d;
  const int64_t s = b * b + 2 * 2 * b * KP;
  const int64_t v = 2 * b * bd + b * KP + 2 * KP * bd;
  return s > v ? s : v;
}

template <int D, int B>
hipError_t launch(const void* Q, const void* K, const void* V, float* O, float* lse, int64_t bh,
                  int64_t n, float scale, void* ws, hipStream_t stream) {
  const ScLayout L = sc_layout(bh, n, B);
  char* base = static_cast<char*>(ws);
  bf16* E = reinterpret_cast<bf16*>(base + L.e_off);
  float* mst = reinterpret_cast<float*>(base + L.m_off);
  float* lst = reinterpret_cast<float*>(base + L.l_off);
  const int nt = (int)L.nt, npad = (int)L.npad;
  const float c = scale * kLog2e;

  const int total1 = (int)(bh * L.nt * L.nt);
  hipLaunchKernelGGL((sc_scores_exp<D, B>), dim3(total1), dim3(B * 2), 0, stream,
                     static_cast<const bf16*>(Q), static_cast<const bf16*>(K), E, mst, lst,
                     (int)n, nt, npad, total1, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = bh * n;
  hipLaunchKernelGGL(sc_merge_stats, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                     mst, lst, lse, rows, nt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BD = B < D ? B : D;
  const int total3 = (int)(bh * L.nt * (D / BD));
  hipLaunchKernelGGL((sc_value_product<D, B>), dim3(total3), dim3(B * 2), 0, stream,
                     static_cast<const bf16*>(V), E, mst, O, (int)n, nt, npad, total3);
  return hipGetLastError();
}

}  // namespace

bool smallcache_supported(int64_t d) { return d == 64 || d == 128 || d == 256; }

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
    case 64 * 1000 + 64: return launch<64, 64>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
    case 64 * 1000 + 128: return launch<64, 128>(Q, K, V, O, lse, bh, n, scale, workspace, stream);
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
