// egm_mfma_probe.hip - a measurement kernel, not part of the GEMM library.
//
// Sustained MFMA throughput of the two 16-bit MFMA shapes gfx950 offers for a
// 32-row accumulator tile: v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16.
// Every wave runs a long chain of independent MFMAs on operands drawn once
// from a per-lane linear congruential generator and rotated between MFMAs
// (so that the multiplier inputs switch as they do in a GEMM), with no memory
// traffic besides one store per lane at the end.  Run back to back on every CU
// while the board's power and clocks are sampled, it shows what each shape
// sustains under the board's power regulation.  Built into its own library
// (libegm_probe.so), which only the benchmark's probe leg loads.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves per workgroup, two per SIMD

// four A and four B operands per lane, values in [-1, 1)
__device__ __forceinline__ void draw_operands(f16x8 (&a)[4], f16x8 (&b)[4]) {
  uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
  for (int q = 0; q < 4; ++q)
    for (int i = 0; i < 8; ++i) {
      h = h * 1664525u + 1013904223u;
      a[q][i] = (_Float16)((float)((int)(h >> 20) - 2048) * (1.0f / 2048.0f));
      h = h * 1664525u + 1013904223u;
      b[q][i] = (_Float16)((float)((int)(h >> 20) - 2048) * (1.0f / 2048.0f));
    }
}

// 8 accumulators of 32x32 (128 registers); 8 MFMAs of 32768 flops per iteration
__global__ void __launch_bounds__(kThreads) mfma_probe_32x32x16(float* out, int iters) {
  f16x8 a[4], b[4];
  draw_operands(a, b);
  f32x16 c[8];
  for (int t = 0; t < 8; ++t)
    for (int e = 0; e < 16; ++e) c[t][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) c[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t & 3], b[(t >> 1) & 3], c[t], 0, 0, 0);
  }
  float s = 0.0f;
  for (int t = 0; t < 8; ++t)
    for (int e = 0; e < 16; ++e) s += c[t][e];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// 32 accumulators of 16x16 (128 registers); 32 MFMAs of 16384 flops per iteration
__global__ void __launch_bounds__(kThreads) mfma_probe_16x16x32(float* out, int iters) {
  f16x8 a[4], b[4];
  draw_operands(a, b);
  f32x4 c[32];
  for (int t = 0; t < 32; ++t)
    for (int e = 0; e < 4; ++e) c[t][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 32; ++t) c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t & 3], b[(t >> 2) & 3], c[t], 0, 0, 0);
  }
  float s = 0.0f;
  for (int t = 0; t < 32; ++t)
    for (int e = 0; e < 4; ++e) s += c[t][e];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// One launch of `blocks` workgroups of 512 lanes on `stream`, each wave doing
// `iters` iterations: 262144 flops per iteration and wave for shape 32 (8
// MFMAs of 32x32x16), 524288 for shape 16 (32 MFMAs of 16x16x32).  out:
// blocks * 512 floats on the device.  Returns 0, or 1 for a bad argument, 2
// for a launch error.  Does not wait for the kernel.
extern "C" int egm_mfma_probe(int shape, int iters, int blocks, float* out, void* stream) {
  if ((shape != 32 && shape != 16) || iters < 1 || blocks < 1 || out == nullptr) return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (shape == 32)
    hipLaunchKernelGGL(mfma_probe_32x32x16, dim3(blocks), dim3(kThreads), 0, s, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_16x16x32, dim3(blocks), dim3(kThreads), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
