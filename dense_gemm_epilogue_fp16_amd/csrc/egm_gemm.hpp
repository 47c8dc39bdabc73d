// egm_gemm.hpp - the fused GEMM + epilogue kernel for gfx950.
//
// One workgroup (4 waves) computes a BM x BN tile of D = epilogue(A.B):
//   * operand streaming: A [BM x 64] and B [64 x BN] k-slabs are read from HBM
//     with 16-byte buffer loads (out-of-range lanes read 0, so ragged edges
//     need no branches), staged in registers one k-slab ahead, and written to
//     a double-buffered LDS ring.  B arrives n-contiguous; each thread
//     transposes its 8-column unit in registers so that LDS holds B^T, i.e.
//     both operands k-contiguous, which is what the MFMA operand layout wants.
//     In LDS each slab is split into 4 k-slices of 16 k-values (32 bytes per
//     row), which is exactly what one MFMA step reads: every fragment address
//     is one per-lane base plus an immediate, and a small swizzle of the two
//     16-byte halves spreads the reads of a wave over all banks.
//   * main loop: v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulators, each wave
//     owning a (BM/2) x (BN/2) sub-tile as FM x FN blocks of 32x32.  The MFMA
//     is fed B^T as its row operand and A as its column operand, so it
//     produces D^T blocks: lane l then holds one row of D (l % 32) and runs of
//     4 consecutive columns, which makes the output and residual accesses
//     8-byte vectors and keeps one lane's mask bits in nibbles.
//   * epilogue, in registers, on the fp32 accumulators: bias (per row or per
//     column), then ReLU / tanh-GELU / residual add, the ReLU mask bits, one
//     round-to-nearest-even conversion, and the store.  The product never goes
//     to memory ([bias-fusion] body: the bias is applied by the same thread
//     block right after the core GEMM; [op-fusion] §三: the residual is added
//     while the producer's output is still in registers).
//
// Pages (cited by title):
//   [bias-fusion] "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
//   [op-fusion]   "模型推理中的算子融合优化从LayerNorm到残差连接的图级优化"
#pragma once

#include "egm_device.hpp"

namespace egm {

struct GemmArgs {
  const void* A;     // [M,K]
  const void* B;     // [K,N]
  void* D;           // [M,N] (the workspace P for the first kernel of the two-kernel path)
  const void* bias;  // [M] or [N]
  const void* R;     // [M,N] residual
  void* aux;         // [M,N/8] mask bytes
  int32_t M, N, K;
  int32_t bias_layout;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
};

template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NT = 256;
  static constexpr int WM = 2, WN = 2;                    // 2 x 2 waves
  static constexpr int WTM = BM / WM, WTN = BN / WN;      // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;      // 32x32 blocks per wave
  static constexpr int A_LD = BM * 8 / NT;                // 16-byte A chunks per thread per slab
  static constexpr int KR = 8 * BN / NT;                  // k-rows in a thread's 8-column B unit
  static constexpr int KG = BK / KR;                      // B units along k
  // LDS layout of one operand slab: 4 k-slices of 16 k-values; slice s holds,
  // for every row, its 16 k-values (32 bytes) of that slice.  A slice is
  // padded by 32 bytes so that the 4 slices of one row start on different
  // banks (16-byte writes of a row's 8 chunks by 8 lanes are conflict-free).
  static constexpr int PAD = 32;
  static constexpr int A_SLICE = BM * 32 + PAD, B_SLICE = BN * 32 + PAD;
  static constexpr int A_BYTES = 4 * A_SLICE;
  static constexpr int B_BYTES = 4 * B_SLICE;
  static constexpr int LDS_BYTES = 2 * (A_BYTES + B_BYTES);
  static_assert(FM >= 1 && FN >= 1, "tile too small for 2x2 waves of 32x32 blocks");
  static_assert(A_LD >= 1 && (BM * 8) % NT == 0, "A slab does not split over the threads");
  static_assert(KR == 2 || KR == 4 || KR == 8, "B unit must be 2, 4 or 8 k-rows");
};

// Inside a slice a row's two 16-byte halves (k 0-7, k 8-15) swap places when
// bit 2 xor bit 3 of the row is set.  An MFMA operand read has lane l reading
// half (l / 32) of row (base + l % 32): any 8 consecutive rows then cover all
// 32 four-byte banks, and any 16 consecutive rows all 64 of a 64-bank LDS.
__device__ __forceinline__ uint32_t half_swz(uint32_t row) { return ((row >> 2) ^ (row >> 3)) & 1u; }

// byte offset of (row, 16-byte chunk c = 8 k-values) inside one operand slab
template <int SLICE>
__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t c) {
  return (c >> 1) * SLICE + row * 32u + (((c & 1u) ^ half_swz(row)) << 4);
}

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin
// (bid % 8), and each XCD has its own L2: give each XCD one contiguous run of
// a grouped tile order, so the tiles an XCD runs together share A row-panels
// (group_m tile rows) and B column-panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int q = T >> 3, r = T & 7;
  const int x = bid & 7, idx = bid >> 3;
  const int lid = (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
  const int per_group = group_m * tiles_n;
  const int g = lid / per_group;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in = lid - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

template <int DT, int EPI, class C>
__global__ void __launch_bounds__(256, 1) gemm_epilogue_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  uint8_t* const ldsA = smem;                      // 2 stages of A   [BM][64]
  uint8_t* const ldsB = smem + 2 * C::A_BYTES;     // 2 stages of B^T [BN][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int KT = (K + C::BK - 1) / C::BK;

  // ------------------------------------------------------------------ streaming setup
  // A: thread owns chunk ac (8 k-values) of rows ar0 + 32*i.
  const int ac = tid & 7;
  const int ar0 = tid >> 3;
  constexpr int AROWS = C::NT / 8;
  const auto rA = make_rsrc((const uint8_t*)p.A + (size_t)m0 * K * 2, (uint64_t)(M - m0) * K * 2);
  uint32_t aoff[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) aoff[i] = (uint32_t)(ar0 + AROWS * i) * (uint32_t)K * 2u + ac * 16u;

  // B: thread owns a KR x 8 unit: k-rows kg*KR .. +KR-1, columns n0 + cg*8 .. +7.
  const int kg = tid % C::KG;
  const int cg = tid / C::KG;
  const bool bcol_ok = (n0 + cg * 8) < N;
  const uint32_t boff = (uint32_t)(kg * C::KR) * (uint32_t)N * 2u + cg * 16u;

  u32x4 ra[C::A_LD];
  u32x4 rb[C::KR];  // KR rows of 8 columns

  auto gload = [&](int kt) {
    const int kbase = kt * C::BK;
    const bool ak_ok = (kbase + ac * 8) < K;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i)
      ra[i] = buf_load16(rA, ak_ok ? aoff[i] + (uint32_t)kbase * 2u : OOB_OFFSET);
    const uint64_t bstart = (uint64_t)kbase * N + n0;
    const uint64_t bsize = (uint64_t)K * N;
    const auto rB = make_rsrc((const uint8_t*)p.B + (bstart < bsize ? bstart : 0) * 2,
                              bstart < bsize ? (bsize - bstart) * 2 : 0);
#pragma unroll
    for (int r = 0; r < C::KR; ++r)
      rb[r] = buf_load16(rB, bcol_ok ? boff + (uint32_t)r * (uint32_t)N * 2u : OOB_OFFSET);
  };

  auto swrite = [&](uint32_t stage) {
    uint8_t* const sa = ldsA + stage * C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const uint32_t row = ar0 + AROWS * i;
      *(u32x4*)(sa + lds_off<C::A_SLICE>(row, ac)) = ra[i];
    }
    // transpose the KR x 8 unit: column c gets the KR k-values of that column
    uint8_t* const sb = ldsB + stage * C::B_BYTES;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[C::KR / 2];
#pragma unroll
      for (int q = 0; q < C::KR / 2; ++q) {
        const uint32_t lo = rb[2 * q][c >> 1];
        const uint32_t hi = rb[2 * q + 1][c >> 1];
        w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const uint32_t row = cg * 8 + c;
      if constexpr (C::KR == 8) {
        *(u32x4*)(sb + lds_off<C::B_SLICE>(row, kg)) = u32x4{w[0], w[1], w[2], w[3]};
      } else if constexpr (C::KR == 4) {
        *(u32x2*)(sb + lds_off<C::B_SLICE>(row, kg >> 1) + (kg & 1) * 8) = u32x2{w[0], w[1]};
      } else {
        *(uint32_t*)(sb + lds_off<C::B_SLICE>(row, kg >> 2) + (kg & 3) * 4) = w[0];
      }
    }
  };

  // ------------------------------------------------------------------ main loop
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // per-lane fragment bases: row (w?0 + lr), half lh of the k-slice; block i /
  // j and slice ks only add immediates (32*32 bytes per block, one slice each)
  const uint32_t a_lane = (uint32_t)(wm0 + lr) * 32u + (((uint32_t)lh ^ half_swz(lr)) << 4);
  const uint32_t b_lane = (uint32_t)(wn0 + lr) * 32u + (((uint32_t)lh ^ half_swz(lr)) << 4);

  auto compute = [&](uint32_t a_base, uint32_t b_base) {
    const uint8_t* const sa = ldsA + a_base;
    const uint8_t* const sb = ldsB + b_base;
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      u32x4 af[C::FM], bf[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) af[i] = *(const u32x4*)(sa + ks * C::A_SLICE + i * 1024);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bf[j] = *(const u32x4*)(sb + ks * C::B_SLICE + j * 1024);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32<DT>(bf[j], af[i], acc[i][j]);
    }
  };

  // Prologue: slab 0 -> LDS stage 0, slab 1 -> registers.  Steady state: write
  // the registers (slab kt+1) to the other stage, issue the loads of slab kt+2
  // (slabs past K read as zeros and move no data), run the MFMAs on stage kt,
  // one barrier.  The loop body has a single path so the accumulators stay in
  // place across iterations.
  if (KT > 0) {
    gload(0);
    swrite(0);
    gload(1);
    __syncthreads();
    uint32_t cur = 0;
    for (int kt = 0; kt < KT - 1; ++kt) {
      swrite(cur ^ 1u);
      gload(kt + 2);
      compute(a_lane + cur * C::A_BYTES, b_lane + cur * C::B_BYTES);
      __syncthreads();
      cur ^= 1u;
    }
    compute(a_lane + cur * C::A_BYTES, b_lane + cur * C::B_BYTES);
  }

  // ------------------------------------------------------------------ epilogue
  // lane holds D[m0 + wm0 + 32i + lr][n0 + wn0 + 32j + 8g + 4lh + e] = acc[i][j][4g + e]
  const uint32_t rowbytes = (uint32_t)N * 2u;
  const auto rD = make_rsrc((uint8_t*)p.D + (size_t)m0 * N * 2, (uint64_t)(M - m0) * N * 2);
  const auto rR = make_rsrc(EPI == EPI_RESID ? (const uint8_t*)p.R + (size_t)m0 * N * 2 : (const uint8_t*)p.D,
                            EPI == EPI_RESID ? (uint64_t)(M - m0) * N * 2 : 0);

  float bcol[C::FN][4][4];
  if constexpr (EPI != EPI_NONE) {
    if (p.bias_layout == BIAS_COL) {
      const auto rbias = make_rsrc(p.bias, (uint64_t)N * 2);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn0 + 32 * j + 8 * g + 4 * lh;
          const u32x2 v = buf_load8(rbias, col < N ? (uint32_t)col * 2u : OOB_OFFSET);
          bcol[j][g][0] = lo_f32<DT>(v[0]);
          bcol[j][g][1] = hi_f32<DT>(v[0]);
          bcol[j][g][2] = lo_f32<DT>(v[1]);
          bcol[j][g][3] = hi_f32<DT>(v[1]);
        }
    } else {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) bcol[j][g][e] = 0.0f;
    }
  }

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const uint32_t lrow = wm0 + 32 * i + lr;  // row within the tile
    float brow = 0.0f;
    if constexpr (EPI != EPI_NONE) {
      if (p.bias_layout == BIAS_ROW) {
        const auto rbias = make_rsrc(p.bias, (uint64_t)M * 2);
        const int row = m0 + (int)lrow;
        brow = to_f32<DT>(buf_load2(rbias, row < M ? (uint32_t)row * 2u : OOB_OFFSET));
      }
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      uint32_t mword = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn0 + 32 * j + 8 * g + 4 * lh;
        const uint32_t off = col < N ? lrow * rowbytes + (uint32_t)col * 2u : OOB_OFFSET;
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = acc[i][j][4 * g + e];
          if constexpr (EPI != EPI_NONE) z[e] += brow + bcol[j][g][e];
        }
        if constexpr (EPI == EPI_RESID) {
          const u32x2 rv = buf_load8(rR, off);
          z[0] += lo_f32<DT>(rv[0]);
          z[1] += hi_f32<DT>(rv[0]);
          z[2] += lo_f32<DT>(rv[1]);
          z[3] += hi_f32<DT>(rv[1]);
        }
        if constexpr (EPI == EPI_RELU_AUX) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mword |= (z[e] > 0.0f ? 1u : 0u) << (8 * g + 4 * lh + e);
        }
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = activate<EPI>(z[e]);
        buf_store8(u32x2{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3])}, rD, off);
      }
      if constexpr (EPI == EPI_RELU_AUX) {
        // lanes l and l+32 hold complementary nibbles of the same row's 32 columns
        mword |= (uint32_t)__shfl_xor((int)mword, 32);
        const uint32_t mrow = (uint32_t)N / 8u;
        const auto rM = make_rsrc((uint8_t*)p.aux + (size_t)m0 * mrow, (uint64_t)(M - m0) * mrow);
        const int cb = n0 + wn0 + 32 * j;  // first column of the word
        if (lh == (j & 1)) {
          if (cb + 32 <= N && (mrow & 3u) == 0) {
            buf_store4(mword, rM, lrow * mrow + (uint32_t)cb / 8u);
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int c8 = cb + 8 * b;
              buf_store1((uint8_t)(mword >> (8 * b)), rM,
                         c8 < N ? lrow * mrow + (uint32_t)c8 / 8u : OOB_OFFSET);
            }
          }
        }
      }
    }
  }
}

}  // namespace egm
