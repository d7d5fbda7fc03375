// Calibration kernels, for rates this device reaches beside its published
// peaks: a matrix-core loop with no memory traffic (bf16 MFMA rate) and a
// streaming read (HBM read bandwidth).
//
// Every wave runs `iters` rounds of four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (the instruction the attention kernels use) on
// register operands.  The operands are bf16 values in [-amp, amp) from a
// per-lane xorshift sequence; with amp = 0 they are all zero.  The rate
// depends on the data: the card lowers its clock when the matrix core
// toggles many bits.  Four waves per workgroup; each thread writes one float
// (the sum of its accumulators) so the work is not removed.
#include "device_common.h"
#include "launch.h"

namespace at {

__global__ __launch_bounds__(256) void calib_mfma_loop(float* __restrict__ out, int iters,
                                                      float amp) {
  bf16x8 a, b;
  uint32_t x = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 1u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    const float r0 = ((x & 0xffffu) * (1.0f / 32768.0f) - 1.0f) * amp;
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    const float r1 = ((x & 0xffffu) * (1.0f / 32768.0f) - 1.0f) * amp;
    a[i] = (__bf16)r0;
    b[i] = (__bf16)r1;
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma_bf16_32x32x16(a, b, acc[j]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_calib_mfma_loop(float* out, int64_t workgroups, int iters, float amp,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_loop, dim3((unsigned)workgroups), dim3(256), 0, stream, out, iters,
                     amp);
  return hipGetLastError();
}

// Streaming read: thread t of the grid reads the 16-byte chunks t, t + T,
// t + 2T, ... (T threads in the grid) with non-temporal loads, so each
// wave-load covers 1 KB of consecutive memory, and writes the XOR of what
// it read (one word per thread, so the loads are not removed).
__global__ __launch_bounds__(256) void calib_stream_read(const u32x4* __restrict__ src,
                                                        int64_t chunks,
                                                        uint32_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  for (int64_t i = t; i < chunks; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(&src[i]);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[t] = x;
}

hipError_t launch_calib_stream_read(const void* src, int64_t bytes, uint32_t* out,
                                    int64_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(calib_stream_read, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace at
