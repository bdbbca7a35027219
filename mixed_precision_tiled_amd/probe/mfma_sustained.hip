// Sustained dense MFMA throughput of the whole GPU, for the measurement
// harness (not part of the attention library).
//
// Published MFMA peaks assume the top engine clock; under a sustained
// full-chip matrix load the clock settles lower.  This probe keeps every
// SIMD's matrix pipe busy with two waves of four independent 32x32 MFMA
// chains on pseudo-random operands (operand toggling sets the power draw,
// hence the clock) and records, per workgroup, the shader-clock ticks
// (s_memtime) and 100 MHz real-time ticks (s_memrealtime) it ran for.  The
// caller times the launch with events: throughput = ops / time, clock =
// shader ticks / real-time ticks x 100 MHz.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t lcg(uint32_t& s) {
  s = s * 1664525u + 1013904223u;
  return s;
}

// kind 0: bf16 32x32x16 (32768 flop each); kind 1: int8 32x32x32 (65536 op)
template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(uint32_t seed, int iters, float* sink,
                                                         unsigned long long* clk) {
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t s = seed ^ (blockIdx.x * 2654435761u) ^ (threadIdx.x * 40503u);
  float acc = 0.f;
  if constexpr (KIND == 1) {
    i32x4 a, b;
    for (int i = 0; i < 4; ++i) {
      a[i] = (int)lcg(s);
      b[i] = (int)lcg(s);
    }
    i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
      // new operand bits every round (cheap vector ops beside the MFMAs)
      a = a ^ b.yzwx;
      b = b + a.wxyz;
    }
    for (int i = 0; i < 16; ++i) acc += (float)(c0[i] ^ c1[i] ^ c2[i] ^ c3[i]);
  } else {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)((float)(int)(lcg(s) >> 16) * 1e-4f);
      b[i] = (__bf16)((float)(int)(lcg(s) >> 16) * 1e-4f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

// Launches nblk workgroups of 256 threads (four waves), each wave running
// `iters` rounds of four MFMAs of `kind` (0: bf16 32x32x16, 1: int8
// 32x32x32) on `stream`.  sink: nblk * 256 floats, clk: 2 * nblk counters
// (device memory owned by the caller).  Returns 0, or the HIP error code of
// the launch; -1 for invalid arguments.  Operations per launch:
// nblk * 4 * iters * 4 * (32768 for bf16, 65536 for int8).
extern "C" int mfma_probe_launch(int kind, int nblk, int iters, uint32_t seed, float* sink,
                                 unsigned long long* clk, void* stream) {
  if (nblk <= 0 || iters <= 0 || sink == nullptr || clk == nullptr || (kind != 0 && kind != 1))
    return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(nblk), dim3(256), 0, s, seed, iters, sink, clk);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(nblk), dim3(256), 0, s, seed, iters, sink, clk);
  return (int)hipGetLastError();
}
