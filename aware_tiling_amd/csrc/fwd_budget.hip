// Fused streaming forward held to a small on-chip budget, for comparing the
// two schedules at the same M below d^2.
//
// Method: page "The I/O Complexity of Attention, or How Optimal is Flash
// Attention?" (exposition), sections "Softmax without storing the score
// matrix" (the streaming recurrence) and "Large caches: where
// FlashAttention's I/O comes from" (a query block and its accumulators stay
// on chip while every key/value tile streams past; with fast memory M the
// query block has about M/d rows, so K and V are read about N d / M times).
// Below M = d^2 the block cannot be larger than a few dozen rows; this is
// the smallest one the matrix cores take, 32 rows, with 32-key tiles.
//
// One workgroup of four waves per (head, 32-query block).  The 32 query
// rows are shared; wave w owns the d-columns [w d/4, (w+1) d/4) of the Q
// block and of the accumulator U, so each wave holds only a quarter of both.
// Per key tile: every wave forms the partial scores over its d-columns
// (S^T = K Q^T, 32 keys x 32 queries), the four partials meet in LDS and
// every wave adds them in the same order, so all waves run the identical
// softmax (running max with the same lazy rescale as the fused kernel, P in
// bf16, l from the rounded values); then each wave adds P V over its own
// d-columns.  K and V tiles go global -> LDS with direct copies into two
// slots, the next tile in flight while the current one is used.
//
// On-chip elements per workgroup (each counted once whatever its width):
// the Q block and the U block (2 x 32 d), (m, l) per row, two slots each of
// the K and V tiles (4 x 32 d), the four partial score tiles (4 x 32 x 32)
// and the summed score tile (32 x 32): 54,336 at d = 256, below d^2 =
// 65,536.
#include "device_common.h"
#include "launch.h"

namespace at {

namespace {

constexpr int kBudgetRows = 32;  // query rows per workgroup
constexpr int kBudgetKeys = 32;  // keys per K/V tile
constexpr float kBudgetTau = 8.0f;  // lazy rescale threshold (base-2 units)

template <int D>
struct BudgetCfg {
  static constexpr int NW = 4, NT = NW * 64;
  static constexpr int DW = D / NW;                  // d-columns per wave
  static constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int TCH = kBudgetKeys * CPR;      // chunks per tile and tensor
  static constexpr int LI = TCH / NT;                // copies per lane per tile and tensor
  static constexpr int TILE = kBudgetKeys * D;       // bf16 elements per tile
  static_assert(TCH % NT == 0 && DW % 32 == 0, "tile shape");
  static constexpr int64_t ONCHIP = 2LL * kBudgetRows * D + 2 * kBudgetRows +
                                    4LL * kBudgetKeys * D + 4LL * kBudgetRows * kBudgetKeys +
                                    (int64_t)kBudgetRows * kBudgetKeys;
};

// Direct global -> LDS copy of 16 bytes per lane, from inline assembly (the
// compiler then adds no wait for these copies before LDS reads; the kernel
// waits for them itself before each barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0: only LDS copies use it here
__device__ __forceinline__ void budget_copy16(const void* gsrc, bf16* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
      __attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds_wave_base)));
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void budget_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void fwd_budget_kernel(const bf16* __restrict__ Q,
                                                         const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V,
                                                         float* __restrict__ O,
                                                         float* __restrict__ lse, int n, int nqb,
                                                         int total, float c) {
  using C = BudgetCfg<D>;
  constexpr int BC = kBudgetKeys, DW = C::DW;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][C::TILE];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][C::TILE];
  __shared__ __attribute__((aligned(16))) float Sp[C::NW][16 * 64];  // partials, register-major

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int tile = xcd_remap(blockIdx.x, total);
  const int head = tile / nqb;
  const int qblk = tile - head * nqb;
  const size_t hoff = (size_t)head * n * D;
  const bf16* Kh = K + hoff;
  const bf16* Vh = V + hoff;
  const int q = qblk * kBudgetRows + li;
  const int d0 = wave * DW;  // this wave's first d-column

  // Q columns [d0, d0 + DW) of the lane's query as MFMA B operands.
  bf16x8 qreg[DW / 16];
#pragma unroll
  for (int kk = 0; kk < DW / 16; ++kk)
    qreg[kk] = q < n ? *reinterpret_cast<const bf16x8*>(Q + hoff + (size_t)q * D + d0 +
                                                        kk * 16 + 8 * h)
                     : bf16x8{};

  // Copy tile j of K (row-major, chunk swizzle) and V (row-major, transposed
  // read swizzle) into slot j & 1; rows past n are clamped (masked below).
  auto issue = [&](int j) {
    const int slot = j & 1;
#pragma unroll
    for (int it = 0; it < C::LI; ++it) {
      const int p0 = (wave * C::LI + it) * 64;
      const int p = p0 + lane;
      const int row = p / C::CPR, phys = p % C::CPR;
      const int key = min(j * BC + row, n - 1);
      budget_copy16(Kh + (size_t)key * D + (phys ^ chunk_swizzle<D * 2>(row)) * 8,
                    &Ks[slot][p0 * 8]);
      budget_copy16(Vh + (size_t)key * D + (phys ^ vtr_swizzle<D * 2>(row)) * 8,
                    &Vs[slot][p0 * 8]);
    }
  };

  f32x16 uacc[DW / 32];
#pragma unroll
  for (int db = 0; db < DW / 32; ++db) uacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const int nt = (n + BC - 1) / BC;
  const int G = lane >> 4, sl = lane & 15, hh = G >> 1;

  issue(0);
  for (int j = 0; j < nt; ++j) {
    const int slot = j & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this lane's copies of tile j landed
    budget_barrier();               // every lane's; and step j - 1 fully done
    if (j + 1 < nt) issue(j + 1);   // into the slot step j - 1 used

    // partial scores over this wave's d-columns: S^T (keys x queries)
    const bf16* Kt = Ks[slot];
    f32x16 sp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < DW / 16; ++kk) {
      const int chunk = (d0 + kk * 16) / 8 + h;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          Kt + li * D + ((chunk ^ chunk_swizzle<D * 2>(li)) * 8));
      sp = mfma_bf16_32x32x16(a, qreg[kk], sp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Sp[wave][r * 64 + lane] = sp[r];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the partials are written
    budget_barrier();
    f32x16 s = f32x16{};
#pragma unroll
    for (int w = 0; w < C::NW; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] += Sp[w][r * 64 + lane];

    // keys past n in the last tile do not exist
    if (j == nt - 1 && (n % BC) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j * BC + 8 * (r >> 2) + 4 * h + (r & 3) >= n) s[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mc = mx * c;
    const bool need = mc > m + kBudgetTau;
    const float mn = need ? mc : m;
    const float alpha = need ? fast_exp2(m - mn) : 1.0f;
    m = mn;
    float lsum = l * alpha;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const uint32_t pp = pack_bf16x2(fast_exp2(__builtin_fmaf(s[r], c, -m)),
                                      fast_exp2(__builtin_fmaf(s[r + 1], c, -m)));
      pk[r >> 1] = pp;
      lsum = add_bf16x2(pp, lsum);
    }
    l = lsum;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int db = 0; db < DW / 32; ++db) uacc[db] *= alpha;
    }

    // U^T[d0 .., queries] += V^T P^T over the tile's keys; the transposed V
    // reads give the key order of the score accumulator (lane group G
    // covers d rows 16 (G & 1) .. +15 of a 32-row block and key half hh)
    const bf16* Vt = Vs[slot];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 pb =
          __builtin_bit_cast(bf16x8, (u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2],
                                            pk[4 * half + 3]}));
#pragma unroll
      for (int db = 0; db < DW / 32; ++db) {
        u32x2 part[2];
#pragma unroll
        for (int piece = 0; piece < 2; ++piece) {
          const int row = 16 * half + 8 * piece + 4 * hh + (sl >> 2);
          const int dc = d0 + db * 32 + 16 * (G & 1) + 4 * (sl & 3);
          const int phys = (dc >> 3) ^ vtr_swizzle<D * 2>(row);
          part[piece] = lds_read_tr16(Vt + row * D + phys * 8 + (dc & 7));
        }
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, (u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}));
        uacc[db] = mfma_bf16_32x32x16(a, pb, uacc[db]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS may outlive the workgroup

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  if (q < n) {
    float* Or = O + hoff + (size_t)q * D + d0;
#pragma unroll
    for (int db = 0; db < DW / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {uacc[db][4 * g] * inv, uacc[db][4 * g + 1] * inv,
                         uacc[db][4 * g + 2] * inv, uacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Or + db * 32 + 8 * g + 4 * h) = v;
      }
    if (wave == 0 && h == 0 && lse != nullptr)
      lse[(size_t)head * n + q] = (m + __log2f(lt)) * kLn2;
  }
}

bool fused_budget_supported(int64_t d) { return d == 128 || d == 256; }

int64_t fused_budget_onchip(int64_t d) {
  switch (d) {
    case 128: return BudgetCfg<128>::ONCHIP;
    case 256: return BudgetCfg<256>::ONCHIP;
    default: return 0;
  }
}

hipError_t launch_fwd_budget_bf16(const void* Q, const void* K, const void* V, float* O,
                                  float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                                  hipStream_t stream) {
  const int nqb = (int)((n + kBudgetRows - 1) / kBudgetRows);
  const int total = (int)(bh * nqb);
  const float c = scale * kLog2e;
  const bf16* q = static_cast<const bf16*>(Q);
  const bf16* k = static_cast<const bf16*>(K);
  const bf16* v = static_cast<const bf16*>(V);
  switch (d) {
    case 128:
      hipLaunchKernelGGL(fwd_budget_kernel<128>, dim3(total), dim3(256), 0, stream, q, k, v, O,
                         lse, (int)n, nqb, total, c);
      break;
    case 256:
      hipLaunchKernelGGL(fwd_budget_kernel<256>, dim3(total), dim3(256), 0, stream, q, k, v, O,
                         lse, (int)n, nqb, total, c);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace at
