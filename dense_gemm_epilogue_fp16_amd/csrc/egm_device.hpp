// egm_device.hpp - device-side building blocks shared by the fused GEMM kernel
// and the stand-alone epilogue kernel: vector types, buffer resources, 16-bit
// conversions and the epilogue functions applied to fp32 accumulators.
//
// Pages (cited by title):
//   [bias-fusion] "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
//   [op-fusion]   "模型推理中的算子融合优化从LayerNorm到残差连接的图级优化"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace egm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum DType { DT_F16 = 0, DT_BF16 = 1 };

// Epilogue kinds (device side).  EPI_NONE stores the bare product (the DEFAULT
// epilog, and the first kernel of the two-kernel path).  EPI_DRELU and
// EPI_DRELU_BGRAD are the backward epilogues: the product is the gradient at
// the ReLU output, kept where the forward mask bit is set (and, for BGRAD,
// also summed along the forward bias's broadcast axis).
enum Epi {
  EPI_NONE = 0,
  EPI_BIAS = 1,
  EPI_RELU = 2,
  EPI_GELU = 3,
  EPI_RELU_AUX = 4,
  EPI_RESID = 5,
  EPI_DRELU = 6,
  EPI_DRELU_BGRAD = 7
};
constexpr bool epi_adds_bias(int epi) { return epi >= EPI_BIAS && epi <= EPI_RESID; }
constexpr bool epi_reads_mask(int epi) { return epi == EPI_DRELU || epi == EPI_DRELU_BGRAD; }
enum BiasLayout { BIAS_NONE = 0, BIAS_ROW = 1, BIAS_COL = 2 };

// ---------------------------------------------------------------------------
// Buffer resources.  Out-of-range lanes of a raw buffer load read 0 and
// out-of-range lanes of a buffer store are dropped, so edge tiles need no
// branches: a lane whose element lies outside the matrix gets OOB_OFFSET.
// ---------------------------------------------------------------------------
constexpr uint32_t OOB_OFFSET = 0x80000000u;
constexpr uint32_t MAX_RECORDS = 0x7ffffff0u;  // keeps OOB_OFFSET out of range
constexpr int RSRC_FLAGS = 0x00020000;         // 32-bit data format, raw addressing

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > MAX_RECORDS ? MAX_RECORDS : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, RSRC_FLAGS);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store1(uint8_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// 16-bit <-> fp32.  Widening is exact; narrowing rounds to nearest-even (the
// hardware conversion under the default rounding mode).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (DT == DT_F16) {
    return (float)__builtin_bit_cast(_Float16, h);
  } else {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
  }
}

// widen the low / high 16 bits of a packed pair
template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w) { return to_f32<DT>((uint16_t)(w & 0xffffu)); }
template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w) { return to_f32<DT>((uint16_t)(w >> 16)); }

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == DT_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// ---------------------------------------------------------------------------
// MFMA 32x32x16, fp32 accumulate.  a: 8 values of the row operand, b: 8 values
// of the column operand (both k-contiguous per lane).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// MFMA 16x16x32, fp32 accumulate: a and b hold 8 consecutive k-values of the
// row (column) l % 16, k-values 8 (l / 16) .. +7; lane l receives rows
// 4 (l / 16) .. +3 of column l % 16.  Same k per register position in both
// operands is all the sum needs.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// fp8 operands: v_mfma_f32_32x32x64_f8f6f4, 64 k-values per instruction.
// Each operand is 32 bytes per lane: lane l holds row (column) l % 32 and the
// k-values 32 (l / 32) .. +31 in byte order (checked on the GPU with an
// in-bounds probe against a host product, all four format pairs).  FA / FB
// select the format of the first / second operand: 0 E4M3, 1 E5M2.  The
// scaled form of the builtin with zero scale operands is the plain
// instruction (no block scaling).
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma32_f8(u32x8 a, u32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                         c, FA, FB, 0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Epilogue arithmetic on fp32 (before the single rounding to 16 bits).
// ---------------------------------------------------------------------------

// tanh-form GELU (Hendrycks & Gimpel; [op-fusion] §一 names GELU in the FFN
// chain).  0.5 z (1 + tanh(u)) equals z * sigmoid(2u) = z / (1 + e^{-2u}),
// u = sqrt(2/pi) (z + 0.044715 z^3); e^{-2u} is taken as 2^(-2u log2 e) with the
// hardware exp2, and the division as the hardware reciprocal.  Large |z|
// saturate cleanly: 2^t -> inf gives -0 for z << 0, 2^t -> 0 gives z for z >> 0.
__device__ __forceinline__ float gelu_tanh(float z) {
  constexpr float kC0 = 0.7978845608028654f;   // sqrt(2/pi)
  constexpr float kC1 = 0.044715f;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float k0 = -2.0f * kC0 * kLog2e;
  constexpr float k1 = k0 * kC1;
  float t = z * __builtin_fmaf(k1, z * z, k0);
  float e = __builtin_amdgcn_exp2f(t);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int EPI>
__device__ __forceinline__ float activate(float z) {
  if constexpr (EPI == EPI_RELU || EPI == EPI_RELU_AUX) {
    return z > 0.0f ? z : 0.0f;
  } else if constexpr (EPI == EPI_GELU) {
    return gelu_tanh(z);
  } else {
    return z;
  }
}

}  // namespace egm
