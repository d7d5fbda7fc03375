// Direct global -> LDS copies issued from inline assembly, exact vmcnt
// waits, and a workgroup barrier without a memory fence (gfx950).
//
// The compiler treats its own global_load_lds builtins as LDS writes it
// cannot tell apart, and makes every later LDS read wait for all of them
// (s_waitcnt vmcnt(0)), which serialises a prefetch of the next tile with
// the reads of the current one.  Copies issued from inline assembly are
// invisible to it: the kernels wait for exactly the copies they need with
// wait_vm<N> before a barrier without a fence.  The compiler's own waits for
// ordinary loads stay correct, since copies it does not count only lengthen
// them.  A kernel that issues these copies ends with wait_vm<0>() so that no
// copy into LDS outlives its workgroup.
#pragma once

#include <cstdint>

#include "device_common.h"

namespace at {

// s_waitcnt with vmcnt = N and the other counters left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0: only LDS copies use it here
// 16 bytes per lane (global_load_lds_dwordx4): lane l's 16 bytes land at
// lds_wave_base + 16 l; lds_wave_base must be uniform across the wave.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
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
// 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes land at
// lds_wave_base + 4 l.
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
      __attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds_wave_base)));
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(gsrc), "s"(lds)
      : "memory", "m0");
}
// LDS byte address of a pointer into a __shared__ array.  Kernels take it
// once per ring (a constant) and add slot and wave offsets as scalars, which
// spares every copy the generic-to-LDS pointer conversion and its null test.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
      reinterpret_cast<const char*>(p));
}

// Buffer resource (V#) for `bytes` bytes from `base`: raw addressing, no
// stride, the range check against `bytes` turning every read past the end
// into zeros.  Built with scalar instructions from a wave-uniform base.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane through a buffer resource (buffer_load_dwordx4 ... lds):
// lane l reads bytes [voff + soff, +16) of the resource (zeros past its end)
// into lds_wave_base + 16 l; soff is wave-uniform (an SGPR).
__device__ __forceinline__ void dma16_buf(rsrc_t rs, uint32_t voff, uint32_t soff,
                                          const void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
      __attribute__((address_space(3))) const char*)(reinterpret_cast<const char*>(lds_wave_base)));
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
      : "memory", "m0");
}
// Copies through a buffer resource with the LDS destination given as a
// wave-uniform LDS byte address (see lds_addr): 16 bytes per lane, the same
// with the nt (non-temporal) policy for data read once (the lines are marked
// for early eviction, so such a stream does not push reused operands out of
// the caches), and 4 bytes per lane (lane l's 4 bytes at lds + 4 l).
__device__ __forceinline__ void dma16_buf_at(rsrc_t rs, uint32_t voff, uint32_t soff,
                                             uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
      : "memory", "m0");
}
__device__ __forceinline__ void dma16_buf_nt_at(rsrc_t rs, uint32_t voff, uint32_t soff,
                                                uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
      : "memory", "m0");
}
__device__ __forceinline__ void dma4_buf_at(rsrc_t rs, uint32_t voff, uint32_t soff,
                                            uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that frees a ring slot for the next copies, without a
// full memory fence: every lane has already waited for its own copies with
// an exact vmcnt, and later copies stay in flight across it (a fence would
// wait for them).  It does wait for this wave's own LDS reads
// (lgkmcnt(0)): the compiler may issue a step's last reads before the
// barrier and consume them after it, and s_barrier alone does not wait for
// them, so another wave could start a copy into the slot they still read.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void slot_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unchanged
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace at
