// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, bf16 packing, LDS reads and copies.  The integer index maps
// (swizzles, offsets) are in index_maps.h.
//
// MFMA operand layouts used throughout (wave64, lane l, h = l / 32, i = l % 32):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[i][8h .. 8h+7]      (8 bf16, k contiguous)
//     B: lane l holds B[8h .. 8h+7][i]      (8 bf16, k contiguous)
//     D: lane l, register r holds D[8(r/4) + 4h + r%4][i]
//   v_mfma_f32_32x32x2_f32    D[32x32] += A[32x2] * B[2x32]
//     A: lane l holds A[i][h];  B: lane l holds B[h][i];  D as above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "index_maps.h"

namespace at {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const bf16x8& a, const bf16x8& b,
                                                     const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// fp32 sum of the two bf16 halves of `p` added to `acc` (v_dot2c_f32_bf16
// against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// v_perm_b32 selectors building {lo16(a), lo16(b)} and {hi16(a), hi16(b)}
// (a in the low half of the result).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x, x of lane l ^ 32) in every lane, with one v_permlane32_swap_b32
// (which exchanges lanes 32..63 of its first operand with lanes 0..31 of
// its second) instead of a ds_bpermute round trip through the LDS unit.
// With both operands holding x, lane i < 32 ends with {x[i], x[i + 32]}
// and lane i >= 32 with {x[i - 32], x[i]}, so one fmaxf finishes the pair.
// Issued from inline assembly (two wait states before and after it) since
// the compiler builtin returns the same register for both results here.
// The max is taken in the same assembly block (v_max_f32: the larger
// operand, the other one if one is a quiet NaN), which spares the compiler's
// NaN canonicalisation of two values it cannot see into.
__device__ __forceinline__ float pair_max_xor32(float x) {
  float a = x, b = x;
  asm volatile(
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(a), "+v"(b));
  return a;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_wave_base + 16 l.  lds_wave_base must be
// uniform across the wave.
__device__ __forceinline__ void load_lds_16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes
// land at lds_wave_base + 4 l.
__device__ __forceinline__ void load_lds_4(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   4, 0, 0);
}

// Four bf16 of a transposed LDS read (ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane i receives element (i mod 4) of the 8 bytes addressed by
// lanes 4e + i/4, for e = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(
          (__attribute__((address_space(3))) char*)(const_cast<bf16*>(p))));
  return __builtin_bit_cast(u32x2, v);
}

}  // namespace at
