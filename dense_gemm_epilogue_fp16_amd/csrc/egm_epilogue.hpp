// egm_epilogue.hpp - stand-alone epilogue kernel: the second launch of the
// deliberately unfused two-kernel path, kept only to measure what fusion saves
// (one extra write + read of the product and one extra launch;
// [bias-fusion] body, opening paragraph: frameworks run the GEMM and the bias
// add as separate kernels, costing a redundant global read and write).
//
// Reads P = round(A.B) (16-bit, [M,N]), the bias and the residual; applies the
// same fp32 epilogue as the fused kernel to fp32(P) + bias; writes D and the
// packed ReLU mask.  Each thread handles runs of 8 columns of one row: one
// 16-byte load of P (and of R), one 16-byte store of D and one mask byte.  The
// backward DRELU reads the mask byte instead and keeps P where its bits are
// set; the bias gradient of the two-kernel path is then summed from D by
// axis_partials_kernel and bias_grad_finish_kernel (the latter also finishes
// the fused kernel's per-block sums).
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
    if constexpr (epi_adds_bias(EPI)) {
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
    if constexpr (epi_reads_mask(EPI)) {
      const uint32_t keep = aux[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = ((keep >> e) & 1u) ? z[e] : 0.0f;
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

// Bias gradient of the two-kernel path, first step: partial sums of D
// ([M,N], the operand dtype) over 32-row or 32-column blocks (the fused kernel
// writes the same layout with whole tiles as the blocks),
//   (1,n) bias (BIAS_COL): partial[rb * N + c] = sum of D[32 rb .. 32 rb + 31, c]
//   (m,1) bias (BIAS_ROW): partial[cb * M + r] = sum of D[r, 32 cb .. 32 cb + 31]
// one thread per (32-row block, 8 columns) or (row, 32-column block).
template <int DT>
__global__ void __launch_bounds__(256) axis_partials_kernel(const void* Dp, int64_t M, int32_t N, int32_t layout,
                                                            float* partial) {
  const uint16_t* D = (const uint16_t*)Dp;
  if (layout == BIAS_COL) {
    const int64_t groups = N / 8, blocks = (M + 31) / 32;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < blocks * groups;
         u += (int64_t)gridDim.x * blockDim.x) {
      const int64_t rb = u / groups, c = (u - rb * groups) * 8;
      float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int64_t r_end = rb * 32 + 32 < M ? rb * 32 + 32 : M;
      for (int64_t r = rb * 32; r < r_end; ++r) {
        const u32x4 v = *(const u32x4*)(D + r * N + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[2 * e] += lo_f32<DT>(v[e]);
          s[2 * e + 1] += hi_f32<DT>(v[e]);
        }
      }
      float* out = partial + rb * N + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = s[e];
    }
  } else {
    const int64_t cblocks = (N + 31) / 32;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < M * cblocks;
         u += (int64_t)gridDim.x * blockDim.x) {
      const int64_t cb = u / M, r = u - cb * M;  // consecutive threads: consecutive rows
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = cb * 32 + 8 * q;
        if (c < N) {
          const u32x4 v = *(const u32x4*)(D + r * N + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) s += lo_f32<DT>(v[e]) + hi_f32<DT>(v[e]);
        }
      }
      partial[cb * M + r] = s;
    }
  }
}

// Bias gradient, last step (both paths): out[x] = sum over c of
// partial[c * len + x].  A workgroup takes 64 consecutive x; its four waves
// each add every fourth chunk (wave q: chunks q, q + 4, ...) in order, and the
// four sums are joined in a fixed order, so the result does not depend on the
// launch.  (A template only so that every unit including this header may see
// it; it is instantiated once, for float.)
template <typename F>
__global__ void __launch_bounds__(256) bias_grad_finish_kernel(const F* partial, int64_t chunks, int64_t len,
                                                               F* out) {
  __shared__ F sums[4][64];
  const int xl = threadIdx.x & 63, q = threadIdx.x >> 6;
  for (int64_t x0 = (int64_t)blockIdx.x * 64; x0 < len; x0 += (int64_t)gridDim.x * 64) {
    const int64_t x = x0 + xl;
    F s = 0;
    if (x < len) {
#pragma unroll 8
      for (int64_t c = q; c < chunks; c += 4) s += partial[c * len + x];
    }
    sums[q][xl] = s;
    __syncthreads();
    if (q == 0 && x < len) out[x] = (sums[0][xl] + sums[1][xl]) + (sums[2][xl] + sums[3][xl]);
    __syncthreads();
  }
}

}  // namespace egm
