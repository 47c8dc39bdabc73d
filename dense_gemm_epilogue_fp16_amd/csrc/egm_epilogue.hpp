// egm_epilogue.hpp - stand-alone epilogue kernel: the second launch of the
// deliberately unfused two-kernel path, kept only to measure what fusion saves
// (one extra write + read of the product and one extra launch;
// [bias-fusion] body, opening paragraph: frameworks run the GEMM and the bias
// add as separate kernels, costing a redundant global read and write).
//
// Reads P = round(A.B) (16-bit, [M,N]), the bias and the residual; applies the
// same fp32 epilogue as the fused kernel to fp32(P) + bias; writes D and the
// packed ReLU mask.  Each thread handles runs of 8 columns of one row: one
// 16-byte load of P (and of R), one 16-byte store of D and one mask byte.
//
// Pages (cited by title):
//   [bias-fusion] "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
#pragma once

#include "egm_device.hpp"

namespace egm {

struct EpiArgs {
  const void* P;     // [M,N] product, rounded to the operand dtype
  const void* bias;  // [M] or [N]
  const void* R;     // [M,N] residual
  void* D;           // [M,N]
  void* aux;         // [M,N/8]
  int64_t M;
  int32_t N;
  int32_t bias_layout;
};

template <int DT, int EPI>
__global__ void __launch_bounds__(256) epilogue_kernel(EpiArgs p) {
  const int64_t per_row = p.N / 8;
  const int64_t units = p.M * per_row;
  const uint16_t* P = (const uint16_t*)p.P;
  const uint16_t* bias = (const uint16_t*)p.bias;
  const uint16_t* R = (const uint16_t*)p.R;
  uint16_t* D = (uint16_t*)p.D;
  uint8_t* aux = (uint8_t*)p.aux;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / per_row;
    const int64_t col = (u - row * per_row) * 8;
    const int64_t idx = row * p.N + col;
    const u32x4 pv = *(const u32x4*)(P + idx);
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[2 * e] = lo_f32<DT>(pv[e]);
      z[2 * e + 1] = hi_f32<DT>(pv[e]);
    }
    if constexpr (EPI != EPI_NONE) {
      if (p.bias_layout == BIAS_ROW) {
        const float b = to_f32<DT>(bias[row]);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += b;
      } else {
        const u32x4 bv = *(const u32x4*)(bias + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[2 * e] += lo_f32<DT>(bv[e]);
          z[2 * e + 1] += hi_f32<DT>(bv[e]);
        }
      }
    }
    if constexpr (EPI == EPI_RESID) {
      const u32x4 rv = *(const u32x4*)(R + idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[2 * e] += lo_f32<DT>(rv[e]);
        z[2 * e + 1] += hi_f32<DT>(rv[e]);
      }
    }
    if constexpr (EPI == EPI_RELU_AUX) {
      uint32_t bits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) bits |= (z[e] > 0.0f ? 1u : 0u) << e;
      aux[u] = (uint8_t)bits;
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack2<DT>(activate<EPI>(z[2 * e]), activate<EPI>(z[2 * e + 1]));
    *(u32x4*)(D + idx) = out;
  }
}

}  // namespace egm
