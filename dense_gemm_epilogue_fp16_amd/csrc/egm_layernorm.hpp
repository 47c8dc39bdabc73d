// egm_layernorm.hpp - LayerNorm over rows, the normalisation that follows the
// FFN down-projection ([op-fusion] §二):
//   y = (x - mean) / sqrt(var + eps) * gamma + beta (+ r)
// with mean and the biased variance taken over each row of length N, gamma and
// beta per column, and an optional residual r added to the normalised output
// (the page's LayerNorm + residual variant).  It cannot be a GEMM epilogue
// unless one tile spans a whole row, so it is its own kernel, one HBM pass:
//   * TPR threads own a row (64: one wave; 256: a workgroup); thread t holds
//     the 16-byte chunks t, t + TPR, ... of the row in registers (consecutive
//     lanes read consecutive 16 bytes), so x is read once and y written once;
//   * statistics in one pass over the registers ([op-fusion] §二: Welford's
//     online method): each chunk's 8 values give a (count, mean, M2) triple,
//     merged chunk by chunk and then across threads with the pairwise update
//     n = na + nb, mean = ma + d nb / n, M2 = Ma + Mb + d^2 na nb / n
//     (d = mb - ma), always with the lower-numbered partner as "a", so every
//     thread of a row ends with the same mean and M2;
//   * rstd = 1 / sqrt(M2 / N + eps); each value is normalised, scaled, shifted
//     (plus the residual) in fp32 and rounded once to the 16-bit type;
//   * rows owned by a whole workgroup load gamma and beta together with x.
// Columns past N (a ragged last chunk cannot occur: N is a multiple of 8)
// read as absent; rows past M are not touched.
//
// Pages (cited by title):
//   [op-fusion] "模型推理中的算子融合优化从LayerNorm到残差连接的图级优化"
#pragma once

#include "egm_device.hpp"

namespace egm {

struct LnArgs {
  const void* x;      // [M, N]
  const void* r;      // [M, N] residual or nullptr
  const void* gamma;  // [N] or nullptr (1)
  const void* beta;   // [N] or nullptr (0)
  void* y;            // [M, N]; may be x (every thread reads its chunks before any write)
  float* mean;        // [M] or nullptr
  float* rstd;        // [M] or nullptr
  int64_t M;
  int32_t N;
  float eps;
};

struct Welford {
  float n, mean, m2;
};

// the pairwise update (a is the lower-numbered side, so the result is the same
// whichever partner computes it)
__device__ __forceinline__ Welford welford_merge(const Welford& a, const Welford& b) {
  const float n = a.n + b.n;
  if (n == 0.0f) return a;
  const float d = b.mean - a.mean;
  const float wb = b.n / n;
  return Welford{n, a.mean + d * wb, a.m2 + b.m2 + d * d * a.n * wb};
}

template <int DT, int TPR, int CPT, bool RES>
__global__ void __launch_bounds__(256) layernorm_kernel(LnArgs p) {
  constexpr int RPW = 256 / TPR;  // rows per workgroup
  const int t = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const int N = p.N;
  const int chunks = N / 8;
  const bool live = row < p.M;
  const uint64_t row_bytes = (uint64_t)N * 2;
  const auto rx = make_rsrc((const uint8_t*)p.x + (live ? row : 0) * row_bytes, live ? row_bytes : 0);
  const auto rr = make_rsrc(RES ? (const uint8_t*)p.r + (live ? row : 0) * row_bytes : (const uint8_t*)p.x,
                            RES && live ? row_bytes : 0);

  // load: chunk c = t + TPR q covers columns 8c .. 8c+7
  u32x4 v[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = t + TPR * q;
    v[q] = buf_load16(rx, c < chunks ? (uint32_t)c * 16u : OOB_OFFSET);
  }
  // gamma and beta: rows of a whole workgroup (256 threads) load theirs with
  // x, so that their latency is not paid again after the statistics (about
  // 8 % of a 65536 x 16384 bf16 pass); the shorter rows (a wave each, several
  // rows per workgroup) keep more rows in flight without the extra registers
  // and load them after the statistics
  constexpr bool kGbEarly = TPR == 256 && CPT <= 8;
  u32x4 gve[kGbEarly ? CPT : 1], bve[kGbEarly ? CPT : 1];
  if constexpr (kGbEarly) {
    const auto rg0 = make_rsrc(p.gamma != nullptr ? p.gamma : p.x, p.gamma != nullptr ? row_bytes : 0);
    const auto rb0 = make_rsrc(p.beta != nullptr ? p.beta : p.x, p.beta != nullptr ? row_bytes : 0);
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = t + TPR * q;
      const uint32_t off = c < chunks ? (uint32_t)c * 16u : OOB_OFFSET;
      gve[q] = p.gamma != nullptr ? buf_load16(rg0, off) : u32x4{0, 0, 0, 0};
      bve[q] = p.beta != nullptr ? buf_load16(rb0, off) : u32x4{0, 0, 0, 0};
    }
  }
  u32x4 rv[CPT];
  if constexpr (RES) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = t + TPR * q;
      rv[q] = buf_load16(rr, c < chunks ? (uint32_t)c * 16u : OOB_OFFSET);
    }
  }

  // per-thread statistics: each chunk's two-pass mean and M2 over its 8
  // values (in registers), merged into the running triple
  Welford w{0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = t + TPR * q;
    if (c < chunks) {
      float xs[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xs[2 * e] = lo_f32<DT>(v[q][e]);
        xs[2 * e + 1] = hi_f32<DT>(v[q][e]);
      }
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += xs[e];
      const float cm = s * 0.125f;
      float m2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m2 += (xs[e] - cm) * (xs[e] - cm);
      w = welford_merge(w, Welford{8.0f, cm, m2});
    }
  }
  // across the row's threads: butterfly within the wave (partners 1, 2, .. 32
  // or the row's 64 lanes), then the waves of a 256-thread row through LDS
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 1; s < (TPR < 64 ? TPR : 64); s <<= 1) {
    const Welford o{__shfl_xor(w.n, s), __shfl_xor(w.mean, s), __shfl_xor(w.m2, s)};
    w = (lane & s) ? welford_merge(o, w) : welford_merge(w, o);
  }
  if constexpr (TPR > 64) {
    __shared__ Welford part[256 / 64];
    const int wave = threadIdx.x / 64;
    if (lane == 0) part[wave] = w;
    __syncthreads();
    w = part[0];
#pragma unroll
    for (int k = 1; k < TPR / 64; ++k) w = welford_merge(w, part[k]);
  }
  const float mean = w.mean;
  const float rstd = 1.0f / __builtin_sqrtf(w.m2 / (float)N + p.eps);
  if (live && t == 0) {
    if (p.mean != nullptr) p.mean[row] = mean;
    if (p.rstd != nullptr) p.rstd[row] = rstd;
  }
  if (!live) return;

  // normalise, scale, shift (+ residual), round once, store
  const auto rg = make_rsrc(p.gamma != nullptr ? p.gamma : p.x, p.gamma != nullptr ? row_bytes : 0);
  const auto rb = make_rsrc(p.beta != nullptr ? p.beta : p.x, p.beta != nullptr ? row_bytes : 0);
  const auto ry = make_rsrc((uint8_t*)p.y + row * row_bytes, row_bytes);
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = t + TPR * q;
    if (c >= chunks) continue;
    const uint32_t off = (uint32_t)c * 16u;
    u32x4 gv, bv;
    if constexpr (kGbEarly) {
      gv = gve[q];
      bv = bve[q];
    } else {
      gv = p.gamma != nullptr ? buf_load16(rg, off) : u32x4{0, 0, 0, 0};
      bv = p.beta != nullptr ? buf_load16(rb, off) : u32x4{0, 0, 0, 0};
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float y0 = (lo_f32<DT>(v[q][e]) - mean) * rstd;
      float y1 = (hi_f32<DT>(v[q][e]) - mean) * rstd;
      if (p.gamma != nullptr) {
        y0 *= lo_f32<DT>(gv[e]);
        y1 *= hi_f32<DT>(gv[e]);
      }
      if (p.beta != nullptr) {
        y0 += lo_f32<DT>(bv[e]);
        y1 += hi_f32<DT>(bv[e]);
      }
      if constexpr (RES) {
        y0 += lo_f32<DT>(rv[q][e]);
        y1 += hi_f32<DT>(rv[q][e]);
      }
      out[e] = pack2<DT>(y0, y1);
    }
    buf_store16(out, ry, off);
  }
}

}  // namespace egm
