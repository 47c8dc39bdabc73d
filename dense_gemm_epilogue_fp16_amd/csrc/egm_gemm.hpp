// egm_gemm.hpp - the fused GEMM + epilogue kernel for gfx950.
//
// One workgroup of WM x WN waves computes a BM x BN tile of D = epilogue(A.B)
// (4 waves, 2 x 2, for the smaller tiles, 2 waves for 32 x 64; 8 waves, 2 x 4
// of 128 x 64, two per SIMD, for 256 x 256, so that one wave's MFMAs issue
// while its partner waits):
//   * operand streaming: A [BM x BK] and B [BK x BN] k-slabs go from HBM
//     straight into LDS with the gfx950 buffer-load-to-LDS instruction (16 bytes
//     per lane, no VGPR staging); out-of-range lanes read 0, so ragged edges
//     need no branches.  The slabs live in a ring of STAGES LDS buffers: a
//     buffer is refilled as soon as every wave has finished reading it, so a
//     slab's loads are issued STAGES-1 slabs before its MFMAs.
//   * LDS layouts: A is row-major, 2*BK bytes per row, its 16-byte chunks
//     XOR-swizzled by row; B stays row-major as it arrives (k rows of BN
//     values), its 16-byte chunks XOR-swizzled by k.  A fragments are read
//     with 16-byte loads; B fragments with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16), which hands each lane 4 consecutive k-values of one
//     column, exactly the MFMA operand layout, so B never needs a transpose
//     pass.
//   * main loop: v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulators, each wave
//     owning a (BM/WM) x (BN/WN) sub-tile as FM x FN blocks of 32x32.  The MFMA
//     gets B as its row operand and A as its column operand, so it produces
//     D^T blocks: lane l holds one row of D (l % 32) and runs of 4 consecutive
//     columns, which makes the output and residual accesses 8-byte vectors and
//     keeps a lane's mask bits in nibbles.  A slab is BK/16 k-slices; each
//     slice's fragments are read while the previous slice's MFMAs run.  After
//     the last slice's reads: one barrier (the next slab is complete and this
//     buffer free), the refill of this buffer, and the next slab's first-slice
//     reads while the last slice's MFMAs run.
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
  void* aux;         // [M,N/8] mask bytes (written by RELU_AUX, read by DRELU / DRELU_BGRAD)
  float* partial;    // DRELU_BGRAD: fp32 partial sums of dZ, one row of them per tile row
                     // ((1,n) bias: [ceil(M/BM), N]) or per tile column ((m,1) bias:
                     // [ceil(N/BN), M])
  const float* scale_a;  // fp8 operands: per-tensor dequantisation scales (one fp32 each;
  const float* scale_b;  // NULL = 1), read once per workgroup
  // strided batches (grid.y problems in one launch): problem z reads A, B, R
  // and writes D, aux at these element (aux: byte) offsets times z
  int64_t stride_a, stride_b, stride_d, stride_aux;
  int32_t M, N, K;
  int32_t bias_layout;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
};

template <int BM_, int BN_, int STAGES_ = 4, int WM_ = 2, int WN_ = 2, int BK_ = 32, int ES_ = 2, int MI_ = 32>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int ES = ES_;                      // operand element bytes: 2 (fp16/bf16) or 1 (fp8)
  static constexpr int MI = MI_;                      // MFMA block: 32 (32x32x16) or 16 (16x16x32, 16-bit only)
  static constexpr int WM = WM_, WN = WN_;            // WM x WN waves
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave (the epilogue's layout)
  static constexpr int FM16 = WTM / 16, FN16 = WTN / 16;  // 16x16 blocks per wave (MI == 16)
  static constexpr int KI = ES == 2 ? (MI == 32 ? 16 : 32) : 64;  // k per MFMA instruction
  static constexpr int NS = BK / KI;                  // k-slices per slab
  static constexpr int CE = 16 / ES;                  // elements per 16-byte chunk
  static constexpr int A_ROW = BK * ES;               // bytes per A row in LDS
  static constexpr int A_CHUNKS = A_ROW / 16;         // 16-byte chunks per A row
  static constexpr int B_ROW = BN * ES;               // bytes per B k-row in LDS
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int B_BYTES = BK * B_ROW;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // one load-to-LDS instruction moves 64 lanes x 16 bytes = 1 KiB
  static constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;
  static constexpr int A_PW = A_DMA / NW, B_PW = B_DMA / NW;  // per wave
  static constexpr int PW = A_PW + B_PW;
  static constexpr int A_ROWS_PER_DMA = 1024 / A_ROW;
  static constexpr int B_CHUNKS = B_ROW / 16;               // 16-byte chunks per B row
  static constexpr int B_ROWS_PER_DMA = 1024 / B_ROW;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid of 32x32 blocks");
  static_assert(ES == 2 ? (BK == 32 || BK == 64) : (ES == 1 && BK == 128), "slabs are 32 or 64 (16-bit) or 128 (fp8) deep");
  static_assert(A_DMA % NW == 0 && B_DMA % NW == 0, "slab must split into whole loads per wave");
  static_assert((STAGES - 1) * PW < 64, "outstanding loads must fit the 6-bit vmcnt");
  // per-wave epilogue stage: 32 rows of the wave tile in T, then 32 mask rows
  static constexpr int EPI_STAGE = 32 * WTN * 2 + 512;
  static_assert(NW * EPI_STAGE <= LDS_BYTES, "epilogue stages must fit in the ring");
  // bias-gradient sums of the waves, combined after the stages: WM rows of BN
  // column sums or WN rows of BM row sums (fp32)
  static constexpr int RED_OFF = NW * EPI_STAGE;
  static_assert(RED_OFF + 4 * (WM * BN > WN * BM ? WM * BN : WN * BM) <= LDS_BYTES, "gradient sums must fit");
  static_assert(BM <= NT && BN <= NT, "one thread per tile row / column for the gradient sums");
  static_assert(STAGES >= 2, "the ring needs a buffer being filled besides the one being read");
  static_assert(LDS_BYTES + 1024 <= 160 * 1024, "LDS ring exceeds 160 KiB");
  static_assert(MI == 32 || (MI == 16 && ES == 2), "16x16 MFMA blocks are built for 16-bit operands");
  // Ring buffer s of A and of B.  32x32 blocks: A and B of a slab side by side
  // (buffer s at s * STAGE_BYTES).  16x16 blocks: all A buffers, then all B
  // buffers, so that a buffer's distance from buffer 0 of its operand stays
  // below the 16-bit offset field of an LDS read (at most 3 x 32 KiB) and the
  // fragment addresses need one register each, whatever the buffer.
  static constexpr uint32_t a_buf(int s) { return MI == 16 ? (uint32_t)(s * A_BYTES) : (uint32_t)(s * STAGE_BYTES); }
  static constexpr uint32_t b_buf(int s) {
    return MI == 16 ? (uint32_t)(STAGES * A_BYTES + s * B_BYTES) : (uint32_t)(s * STAGE_BYTES + A_BYTES);
  }
};

// A: the 16-byte chunks of an A row are XOR-ed with row bits, so that the
// 16-byte fragment reads (16 lanes at a time: consecutive rows, one logical
// chunk) cover all 64 4-byte banks.  64-byte rows (4 chunks): rows r and r+4
// share banks, so the chunk is XOR-ed with bits 2..3; 128-byte rows (8
// chunks): rows r and r+2 share banks, so bits 1..3.  Measured with the
// bank-conflict counter for the 4-chunk case, the other 2-bit row functions
// tried cost 2- to 4-way conflicts.
template <int A_CHUNKS>
__device__ __forceinline__ uint32_t a_swz(uint32_t row) {
  if constexpr (A_CHUNKS == 4) return (row >> 2) & 3u;
  else return (row >> 1) & 7u;
}

// B, 16-bit, 32x32 blocks: chunk index bits 2..3 are XOR-ed with k mod 4, so
// the four k-rows a transposing read touches at once land on different 64-byte
// bank groups.  16-bit, 16x16 blocks: a transposing read takes 32 bytes (one
// block's 16 columns) from each of 8 k-rows per half-wave, k-rows q and q + 8
// (q = 0..3 within a 16-lane group); bits 1..3 of the chunk index are XOR-ed
// with 8 distinct even values, so the 8 pieces cover all 64 banks: k-row bits
// 0..1 and 3 where a k-row spans the 256-byte bank window (rows of 256 or 512
// bytes), bits 1 and 3 where two rows share it (rows of 128 bytes; row parity
// already picks the window half).  fp8: one 8-bit transposing read takes a
// 16-byte chunk pair from 8 consecutive k-rows per half-wave; the pair index
// is XOR-ed with the k-row's position among the rows that share a 256-byte
// bank window, so the 8 pairs cover all 64 banks (rows of 256, 128 or 64
// bytes).  Both 16-bit forms leave k-row bit 2 out, so a block's second
// transposing read (4 k-rows further) keeps the first one's swizzle.
template <int B_CHUNKS, int ES = 2, int MI = 32>
__device__ __forceinline__ uint32_t b_swz(uint32_t krow) {
  if constexpr (ES == 2 && MI == 16) {
    if constexpr (B_CHUNKS >= 16)
      return ((krow & 3u) << 2) | (((krow >> 3) & 1u) << 1);
    else
      return ((((krow >> 1) & 1u) << 2) | (((krow >> 3) & 1u) << 1)) & (B_CHUNKS - 1);
  } else if constexpr (ES == 2) {
    return ((krow & 3u) << 2) & (B_CHUNKS - 1);
  } else {
    constexpr uint32_t RPW = B_CHUNKS >= 16 ? 1 : 16 / B_CHUNKS;  // k-rows per 256-byte window
    return ((krow / RPW) & (B_CHUNKS / 2 - 1)) << 1;
  }
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

// 16-byte global -> LDS copy per lane; lane L lands at lds + 16 L.  Written
// as inline assembly on purpose: the compiler cannot tell which LDS bytes the
// copy writes, and through the builtin it would make every later LDS read wait
// for all copies in flight, which defeats the ring.  The kernel orders the
// copies itself (explicit vmcnt waits before the barrier that publishes a slab).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 make_srd(const void* base, uint64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  // the clamp in 32-bit halves: scalar compares (gfx9 has no 64-bit scalar
  // less-than, and the compiler would merge the halves back into a vector
  // one).  Every caller passes wave-uniform values.
  uint32_t hi = (uint32_t)(bytes >> 32);
  asm("" : "+s"(hi));
  const uint32_t n = hi != 0u || (uint32_t)bytes > MAX_RECORDS ? MAX_RECORDS : (uint32_t)bytes;
  return i32x4{(int32_t)(uint32_t)a, (int32_t)(uint32_t)((a >> 32) & 0xffffu), (int32_t)n, RSRC_FLAGS};
}

// LDS byte address of a __shared__ array (a 32-bit offset into the workgroup's LDS)
__device__ __forceinline__ uint32_t lds_address(uint8_t* shared_array) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)shared_array;
}

__device__ __forceinline__ void dma16(i32x4 srd, uint32_t lds_byte_addr, uint32_t voff) {
  // the LDS address is wave-uniform by construction; make that explicit for M0
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_byte_addr);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  // (an M0 write needs a wait state before a load-to-LDS reads it)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(srd)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i mod 4) of the 4-element rows addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4.
template <int DT>
__device__ __forceinline__ u32x2 lds_read_tr(const uint8_t* p) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  if constexpr (DT == DT_F16) {
    typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
    typedef __attribute__((address_space(3))) h4* hp;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((hp)(lds_ptr)p));
  } else {
    typedef __bf16 b4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
    typedef __attribute__((address_space(3))) b4* bp;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bp)(lds_ptr)p));
  }
}

// 8-bit transposing LDS read: within each 16-lane group, lane i receives byte
// (i mod 8) of the 8-byte rows addressed by lanes i/8, 2 + i/8, .., 14 + i/8,
// in that order (checked on the GPU with an in-bounds probe).
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int i2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i2* lp;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lp)(lds_ptr)p));
}

// s_waitcnt lgkmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
  __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (N << 8) | (0x3 << 14));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// The lane's index in its wave, computed afresh (v_mbcnt).  The epilogue
// takes it from here rather than from threadIdx.x, so that its lane-derived
// offsets are formed after the main loop instead of being kept (or spilled)
// through it.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}


// Cross-lane moves for the bias-gradient sums (VALU only, no LDS traffic).
// swap16(x, y): for each pair of 16-lane rows (0,1), (2,3), the odd row of x
// trades places with the even row of y (v_permlane16_swap); swap32 does the
// same with the two 32-lane halves (v_permlane32_swap).
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                  false, false);
  x = __builtin_bit_cast(float, (uint32_t)r[0]);
  y = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                  false, false);
  x = __builtin_bit_cast(float, (uint32_t)r[0]);
  y = __builtin_bit_cast(float, (uint32_t)r[1]);
}
// DPP lane moves inside a 16-lane row: lane i reads lane i ^ 8 (row_ror:8),
// (i & ~7) | (7 - (i & 7)) (row_half_mirror), i ^ 2 and i ^ 1 (quad_perm)
enum : int { DPP_XOR8 = 0x128, DPP_HALF_MIRROR = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1 };
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Column sums of a 32 x 32 block over its 32 rows.  Lane l holds row l % 32
// and, in v[4g + e], column 8g + 4(l / 32) + e.  Each step pairs every lane
// with a partner that holds the same value indices over other rows; the lane
// keeps one half of its values (chosen by a bit of l that differs from the
// partner's) and adds the partner's copy of that half: 16 -> 8 values over
// rows l, l^16 (row swap), -> 4 over 4 rows (partner l^8), -> 2 (partner in
// the mirrored half-row), -> 1 (partner l^2), then a last add with lane l^1.
// Lane l ends with the sum of v[k], k = (l >> 1) & 15, over all 32 rows.
__device__ __forceinline__ float block_column_sum(float (&v)[16], int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    float x = v[t], y = v[t + 8];
    swap16(x, y);  // even rows now hold (own v[t], partner v[t]), odd rows (partner v[t+8], own v[t+8])
    v[t] = x + y;
  }
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0, b1 = (lane & 2) != 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float give = b3 ? v[t] : v[t + 4], mine = b3 ? v[t + 4] : v[t];
    v[t] = mine + dpp<DPP_XOR8>(give);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float give = b2 ? v[t] : v[t + 2], mine = b2 ? v[t + 2] : v[t];
    v[t] = mine + dpp<DPP_HALF_MIRROR>(give);
  }
  {
    const float give = b1 ? v[0] : v[1], mine = b1 ? v[1] : v[0];
    v[0] = mine + dpp<DPP_XOR2>(give);
  }
  return v[0] + dpp<DPP_XOR1>(v[0]);
}

// ---------------------------------------------------------------------------
// Epilogue on the fp32 accumulators of one wave, then the store.  The
// accumulators come one 32-row block-row at a time from block_row(i, row):
// lane holds D[m0 + wm0 + 32i + lr][n0 + wn0 + 32j + 8g + 4lh + e] = row[j][4g + e]
// ---------------------------------------------------------------------------
template <int DT, int EPI, int WM, int WN, bool SCALED, int FM, int FN, class BlockRow>
__device__ __forceinline__ void epilogue_store(const GemmArgs& p, BlockRow&& block_row, int m0, int n0, int wm0,
                                               int wn0, int lane, uint8_t* stage,
                                               const uint8_t* bias_lds, float* red, float scale) {
  const int M = p.M, N = p.N;
  // The packed outputs of one 32-row block-row go through this wave's private
  // LDS stage so that D leaves as 16-byte row chunks, 4 full rows of the wave
  // tile per store instruction (instead of 8-byte pieces of 32 rows).  Stage
  // rows are ROWB bytes (SLOTS 8-byte slots); slot s of row r sits at slot
  // s ^ xr(r), which makes both the 8-byte writes (32 rows, one slot each) and
  // the 16-byte reads (whole rows) hit distinct banks.
  constexpr int SLOTS = 8 * FN, ROWB = 8 * SLOTS, CH = SLOTS / 2;
  constexpr int RSHIFT = ROWB >= 256 ? 0 : ROWB == 128 ? 1 : 2;  // rows sharing a 256-byte bank window
  auto xr = [](uint32_t r) { return (r >> RSHIFT) & (SLOTS - 1); };
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const uint32_t rowbytes = (uint32_t)N * 2u;
  const auto rD = make_rsrc((uint8_t*)p.D + (size_t)m0 * N * 2, (uint64_t)(M - m0) * N * 2);
  const auto rR = make_rsrc(EPI == EPI_RESID ? (const uint8_t*)p.R + (size_t)m0 * N * 2 : (const uint8_t*)p.D,
                            EPI == EPI_RESID ? (uint64_t)(M - m0) * N * 2 : 0);

  // a (1,n) bias: the tile's BN values sit in LDS (bias_lds), by tile column
  float bcol[FN][4][4];
  if constexpr (epi_adds_bias(EPI)) {
    if (p.bias_layout == BIAS_COL) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 v = *(const u32x2*)(bias_lds + 2 * (wn0 + 32 * j + 8 * g + 4 * lh));
          bcol[j][g][0] = lo_f32<DT>(v[0]);
          bcol[j][g][1] = hi_f32<DT>(v[0]);
          bcol[j][g][2] = lo_f32<DT>(v[1]);
          bcol[j][g][3] = hi_f32<DT>(v[1]);
        }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) bcol[j][g][e] = 0.0f;
    }
  }
  // the packed ReLU mask of a block-row: 32 rows x 4*FN bytes, staged right
  // after the output stage when the wave tile's mask bytes of a row go out as
  // one aligned piece (full-width wave tiles, mask rows a multiple of 4*FN)
  const uint32_t mrow = (uint32_t)N / 8u;
  uint8_t* const mstage = stage + 32 * ROWB;
  const bool mask_rows = n0 + wn0 + 32 * FN <= N && mrow % (4u * FN) == 0;
  // the mask rows of this tile: written by RELU_AUX, read by the backward epilogues
  constexpr bool kMask = EPI == EPI_RELU_AUX || epi_reads_mask(EPI);
  const auto rM = make_rsrc(kMask ? (uint8_t*)p.aux + (size_t)m0 * mrow : (uint8_t*)p.D,
                            kMask ? (uint64_t)(M - m0) * mrow : 0);

  // backward: the forward mask words of the wave tile, all loads issued at
  // once; word (i, j) covers row wm0+32i+lr, columns wn0+32j .. +31 (bit
  // 8g + 4lh + e belongs to this lane's column 8g + 4lh + e)
  uint32_t keep[FM][FN];
  if constexpr (epi_reads_mask(EPI)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = n0 + wn0 + 32 * j;
        const uint32_t mo = (uint32_t)(wm0 + 32 * i + lr) * mrow + (uint32_t)cb / 8u;
        if ((mrow & 3u) == 0) {
          keep[i][j] = buf_load4(rM, mo);  // 4-byte aligned: the word is one load
        } else {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w |= (uint32_t)buf_load1(rM, cb + 8 * b < N ? mo + b : OOB_OFFSET) << (8 * b);
          keep[i][j] = w;
        }
      }
  }
  // the residual: with at most four waves (registers to spare after the main
  // loop) every piece of the wave tile is requested at once, ahead of the
  // block-rows, so that the loads' latency is paid once and not once per
  // block-row (whose stores would otherwise wait behind them); 8-wave tiles
  // load each block-row's pieces with it
  constexpr bool kResidAhead = EPI == EPI_RESID && WM * WN <= 4;
  u32x2 resid[FM][FN][4];
  if constexpr (kResidAhead) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn0 + 32 * j + 8 * g + 4 * lh;
          const uint32_t lrow = wm0 + 32 * i + lr;
          resid[i][j][g] = buf_load8(rR, col < N ? lrow * rowbytes + (uint32_t)col * 2u : OOB_OFFSET);
        }
  }
  // bias gradient: this wave's sums of dZ over its rows, one per column of
  // block j and lane (colacc, (1,n) bias), or over its columns, one per row of
  // block i (rowacc, (m,1) bias); added up in a fixed order
  float colacc[FN], rowacc[FM];
#pragma unroll
  for (int j = 0; j < FN; ++j) colacc[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i) rowacc[i] = 0.0f;

#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t lrow = wm0 + 32 * i + lr;  // row within the tile
    f32x16 acc_row[FN];
    block_row(i, acc_row);
    float brow = 0.0f;
    if constexpr (epi_adds_bias(EPI)) {
      if (p.bias_layout == BIAS_ROW) {
        // range based at the tile's first row: byte offsets stay below 512
        // whatever M is (a range from bias[0] would cap near 2^31 bytes),
        // and rows past M fall outside it and read as 0
        const auto rbias = make_rsrc((const uint8_t*)p.bias + (size_t)m0 * 2, (uint64_t)(M - m0) * 2);
        brow = to_f32<DT>(buf_load2(rbias, lrow * 2u));
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      uint32_t mword = 0;
      // bias gradient sums of this 32 x 32 block: per column (the lane's row
      // only, reduced across the rows below) or per row (the lane's columns,
      // reduced across the two half-waves below)
      float csum[4][4];
      float rsum = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn0 + 32 * j + 8 * g + 4 * lh;
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = acc_row[j][4 * g + e];
          if constexpr (SCALED) z[e] *= scale;  // fp8: the two per-tensor scales, before the bias
          if constexpr (epi_adds_bias(EPI)) z[e] += brow + bcol[j][g][e];
          if constexpr (epi_reads_mask(EPI)) z[e] = ((keep[i][j] >> (8 * g + 4 * lh + e)) & 1u) ? z[e] : 0.0f;
          if constexpr (EPI == EPI_DRELU_BGRAD) {
            csum[g][e] = z[e];
            rsum += z[e];
          }
        }
        if constexpr (EPI == EPI_RESID) {
          const u32x2 rv = kResidAhead ? resid[i][j][g]
                                       : buf_load8(rR, col < N ? lrow * rowbytes + (uint32_t)col * 2u : OOB_OFFSET);
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
        const uint32_t slot = (uint32_t)(8 * j + 2 * g + lh);
        *(u32x2*)(stage + lr * ROWB + ((slot ^ xr(lr)) << 3)) = u32x2{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3])};
      }
      if constexpr (EPI == EPI_DRELU_BGRAD) {
        if (p.bias_layout == BIAS_COL) {
          float v[16];
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * g + e] = csum[g][e];
          colacc[j] += block_column_sum(v, lane);
        } else {
          // sum the block's 32 columns: the two half-waves hold 16 each
          float x = rsum, y = rsum;
          swap32(x, y);  // x: the low half's sum in every lane, y: the high half's
          rowacc[i] += x + y;
        }
      }
      if constexpr (EPI == EPI_RELU_AUX) {
        // lanes l and l+32 hold complementary nibbles of the same row's 32 columns
        mword |= (uint32_t)__shfl_xor((int)mword, 32);
        const int cb = n0 + wn0 + 32 * j;  // first column of the word
        if (mask_rows) {
          if (lh == 0) *(uint32_t*)(mstage + lr * 16 + 4 * j) = mword;
        } else if (lh == (j & 1)) {
          if (cb + 32 <= N && (mrow & 3u) == 0) {
            buf_store4(mword, rM, lrow * mrow + (uint32_t)cb / 8u);
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int c8 = cb + 8 * b;
              buf_store1((uint8_t)(mword >> (8 * b)), rM, c8 < N ? lrow * mrow + (uint32_t)c8 / 8u : OOB_OFFSET);
            }
          }
        }
      }
    }
    if constexpr (EPI == EPI_RELU_AUX) {
      if (mask_rows && lane < 32) {
        const uint32_t moff = (wm0 + 32 * i + lane) * mrow + (uint32_t)(n0 + wn0) / 8u;
        if constexpr (FN == 4) {
          buf_store16(*(const u32x4*)(mstage + lane * 16), rM, moff);
        } else if constexpr (FN == 2) {
          buf_store8(*(const u32x2*)(mstage + lane * 16), rM, moff);
        } else {
          buf_store4(*(const uint32_t*)(mstage + lane * 16), rM, moff);
        }
      }
    }
    // the block-row is staged: write it out as 16-byte row chunks (the same
    // wave wrote it, and a wave's LDS accesses complete in order)
    constexpr int RPI = 1024 / ROWB;  // stage rows per 1 KiB read
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const uint32_t r = q * RPI + lane / CH, m = lane % CH;
      const uint32_t x = xr(r);
      u32x4 v = *(const u32x4*)(stage + r * ROWB + ((((2 * m) ^ x) >> 1) << 4));
      if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      const int col = n0 + wn0 + 8 * (int)m;
      buf_store16(v, rD, col < N ? (wm0 + 32 * i + r) * rowbytes + (uint32_t)col * 2u : OOB_OFFSET);
    }
  }
  if constexpr (EPI == EPI_DRELU_BGRAD) {
    // the tile's sums: the waves that share columns (or rows) leave theirs in
    // LDS, then one thread per tile column (row) adds them in wave order and
    // writes the tile's partial; rows and columns past the matrix hold zeros
    // (their mask bits read as 0) and are not written
    constexpr int BM = WM * 32 * FM, BN = WN * 32 * FN;
    const int tid = (int)threadIdx.x;
    if (p.bias_layout == BIAS_COL) {
      const int wave_m = wm0 / (32 * FM);
      if ((lr & 1) == 0) {
        const int k = (lr >> 1) & 15;
        const int c = 8 * (k >> 2) + 4 * lh + (k & 3);
#pragma unroll
        for (int j = 0; j < FN; ++j) red[wave_m * BN + wn0 + 32 * j + c] = colacc[j];
      }
      __syncthreads();
      if (tid < BN && n0 + tid < N) {
        float t = red[tid];
#pragma unroll
        for (int w = 1; w < WM; ++w) t += red[w * BN + tid];
        p.partial[(size_t)(m0 / BM) * N + n0 + tid] = t;
      }
    } else {
      const int wave_n = wn0 / (32 * FN);
      if (lh == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) red[wave_n * BM + wm0 + 32 * i + lr] = rowacc[i];
      }
      __syncthreads();
      if (tid < BM && m0 + tid < M) {
        float t = red[tid];
#pragma unroll
        for (int w = 1; w < WN; ++w) t += red[w * BM + tid];
        p.partial[(size_t)(n0 / BN) * M + m0 + tid] = t;
      }
    }
  }
}

// DT: the output (and bias / residual) type, and the operand type when F8 is 0.
// F8 = 1 + fa + 2 fb for fp8 operands (fa, fb: 0 E4M3, 1 E5M2 for A and B),
// with C::ES == 1.  BT: B is given transposed, as [N, K] row-major (a linear
// layer's weight); its tile then sits in LDS exactly like A's (K-contiguous
// rows, the same swizzle, the same 16-byte fragment reads), so no
// transposing read is needed.
template <int DT, int EPI, class C, int F8 = 0, bool BT = false>
__global__ void __launch_bounds__(C::NT, 1) gemm_epilogue_kernel(GemmArgs p) {
  static_assert((F8 == 0) == (C::ES == 2), "fp8 kernels use one-byte tiles");
  // the k-slab ring, then the tile's bias slice
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES + 1024];
  uint8_t* const bias_lds = smem + C::LDS_BYTES;
  const uint32_t smem_lds = lds_address(smem);  // the same array as an LDS byte address, for the copies

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int M = p.M, N = p.N, K = p.K;

  if (gridDim.y > 1) {  // problem blockIdx.y of a strided batch
    const int64_t z = blockIdx.y;
    p.A = (const uint8_t*)p.A + z * p.stride_a * C::ES;
    p.B = (const uint8_t*)p.B + z * p.stride_b * C::ES;
    p.D = (uint8_t*)p.D + z * p.stride_d * 2;
    if (p.R != nullptr) p.R = (const uint8_t*)p.R + z * p.stride_d * 2;
    if (p.aux != nullptr) p.aux = (uint8_t*)p.aux + z * p.stride_aux;
  }
  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  // uniform by construction; in scalar registers the tile's buffer ranges and
  // bounds stay scalar arithmetic in the main loop
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int KT = (K + C::BK - 1) / C::BK;

  // A (1,n) bias: wave 0 copies the tile's BN values straight into LDS ahead
  // of the operand loads (its completion is covered by the prologue's wait;
  // lanes past BN/8 write zeros).  A (m,1) bias is read in the epilogue.
  if constexpr (epi_adds_bias(EPI)) {
    if (p.bias_layout == BIAS_COL && wave == 0) {
      const uint32_t c = (uint32_t)n0 + 8u * (uint32_t)lane;  // n is a multiple of 8: whole 16-byte pieces
      dma16(make_srd(p.bias, (uint64_t)N * 2), smem_lds + C::LDS_BYTES,
            lane < C::BN / 8 && c < (uint32_t)N ? c * 2u : OOB_OFFSET);
    }
  }

  // ------------------------------------------------------------------ streaming setup
  // A load q (0 .. A_DMA-1) fills rows R*q .. R*q+R-1 (R = A_ROWS_PER_DMA):
  // lane L -> row R*q + L/A_CHUNKS, physical chunk L%A_CHUNKS, which holds
  // logical chunk (L%A_CHUNKS) ^ a_swz(row).  Offsets are relative to the
  // slab's first column; columns past K read 0.
  // (fp8 tiles of two waves per SIMD, whose main loop uses every register:
  // with B given transposed, the logical chunk of every copy sits in one
  // register, 4 bits each, copy q at bits 4q: k_lc)
  constexpr bool kTight = C::ES == 1 && C::NW == 8;
  // kLean: the 256x256 tile of 8 waves with 16x16x32 blocks.  Its k-slices
  // are 32 deep, so a fragment set is twice that of the 32x32 blocks; only one
  // set of A fragments fits beside the 128 accumulators (see lean_row), and
  // the register tricks of the fp8 tile apply (packed chunk indices for B not
  // transposed, opaque LDS base, no empty refills after the loop, a fresh
  // lane index in the epilogue), plus the copy offsets of off_of.
  constexpr bool kLean = C::MI == 16 && C::NW == 8;
  static_assert(!(kTight || kLean) || C::PW <= 8, "packed chunk indices: at most 8 copies per wave and slab");
  uint32_t a_off[C::A_PW], a_k8[C::A_PW], k_lc = 0;
#pragma unroll
  for (int u = 0; u < C::A_PW; ++u) {
    const uint32_t q = wave * C::A_PW + u;
    const uint32_t row = C::A_ROWS_PER_DMA * q + lane / C::A_CHUNKS;
    const uint32_t lc = (lane % C::A_CHUNKS) ^ a_swz<C::A_CHUNKS>(row);
    a_k8[u] = lc * C::CE;
    if constexpr ((kTight && BT) || (kLean && !BT)) k_lc |= lc << (4 * u);
    a_off[u] = (row * (uint32_t)K + lc * C::CE) * C::ES;
  }
  // B load q fills k-rows q*R .. q*R+R-1 (R = B_ROWS_PER_DMA): lane L -> k-row
  // q*R + L/B_CHUNKS, physical chunk L%B_CHUNKS holding logical chunk
  // (L%B_CHUNKS) ^ b_swz(k-row).  Columns past N read 0; k-rows past K fall
  // outside the slab's buffer range and read 0.
  // Transposed B: load q fills tile rows (n) R*q .. R*q+R-1 as A's loads do;
  // rows past N fall outside the slab's buffer range, columns past K read 0.
  uint32_t b_off[C::B_PW], b_k8[C::B_PW];
#pragma unroll
  for (int u = 0; u < C::B_PW; ++u) {
    const uint32_t q = wave * C::B_PW + u;
    if constexpr (BT) {
      const uint32_t row = C::A_ROWS_PER_DMA * q + lane / C::A_CHUNKS;
      const uint32_t lc = (lane % C::A_CHUNKS) ^ a_swz<C::A_CHUNKS>(row);
      b_k8[u] = lc * C::CE;
      if constexpr ((kTight && BT) || (kLean && !BT)) k_lc |= lc << (4 * (C::A_PW + u));
      b_off[u] = (row * (uint32_t)K + lc * C::CE) * C::ES;
    } else {
      const uint32_t krow = q * C::B_ROWS_PER_DMA + lane / C::B_CHUNKS;
      const uint32_t lc = (lane % C::B_CHUNKS) ^ b_swz<C::B_CHUNKS, C::ES, C::MI>(krow);
      b_k8[u] = 0;
      b_off[u] = (n0 + (int)lc * C::CE < N) ? (krow * (uint32_t)N + lc * C::CE) * C::ES : OOB_OFFSET;
    }
  }

  // Buffer ranges of slab kt (uniform: computed once per slab): A from
  // (m0, kbase) to the end of A, B from (kbase, n0) to the end of B.  Slabs
  // past K get empty ranges: their loads move no data but still count as
  // outstanding, so every slab costs the same vmcnt.
  struct SlabSrd {
    i32x4 a, b;
    uint32_t kbase;
    bool full;  // the whole slab lies below K: the A copies need no per-lane k check
  };
  // The tile's first row (m0 < M) and column (n0 < N) exist, so a slab's start
  // lies inside its operand exactly when kbase < K: one 32-bit scalar compare
  // instead of 64-bit ones (which gfx9 scalar units lack).
  auto slab_srd = [&](int kt) {
    SlabSrd r;
    r.kbase = (uint32_t)kt * C::BK;
    const bool in_k = r.kbase < (uint32_t)K;
    r.full = r.kbase + C::BK <= (uint32_t)K;
    const uint64_t a_start = (uint64_t)m0 * K + r.kbase, a_size = (uint64_t)M * K;
    r.a = make_srd((const uint8_t*)p.A + (in_k ? a_start : 0) * C::ES, in_k ? (a_size - a_start) * C::ES : 0);
    if constexpr (BT) {
      const uint64_t b_start = (uint64_t)n0 * K + r.kbase, b_size = (uint64_t)N * K;
      r.b = make_srd((const uint8_t*)p.B + (in_k ? b_start : 0) * C::ES, in_k ? (b_size - b_start) * C::ES : 0);
    } else {
      const uint64_t b_start = (uint64_t)r.kbase * N + n0, b_size = (uint64_t)K * N;
      r.b = make_srd((const uint8_t*)p.B + (in_k ? b_start : 0) * C::ES, in_k ? (b_size - b_start) * C::ES : 0);
    }
    return r;
  };
  // Load q (0 .. PW-1) of this wave for a slab into ring buffer `stage`: the
  // first A_PW are A loads, the rest B loads.
  // LDS base of the copies.  With one wave per SIMD (4 waves), and in the
  // fp8 tile of two waves per SIMD, the compiler would otherwise hoist every copy's LDS
  // address (one per copy and ring buffer) out of the main loop into
  // registers of their own, and spill them; an opaque base keeps each
  // address a couple of scalar additions at its copy.
  auto copy_base = [&]() {
    uint32_t b = smem_lds;
    if constexpr (C::NW == 4 || kTight || kLean) asm volatile("" : "+s"(b));
    return b;
  };
  // Per-lane k offset of copy u's piece within the slab (A, transposed B);
  // j: the copy's index among this wave's copies of the slab.
  auto k_of = [&](const auto& k8, int u, int j) -> uint32_t {
    if constexpr ((kTight && BT) || (kLean && !BT)) {
      // taken apart at each use (an opaque copy), so that the compiler does
      // not hoist the eight offsets out of the main loop into registers
      uint32_t kl = k_lc;
      asm volatile("" : "+v"(kl));
      return ((kl >> (4 * j)) & 7u) * C::CE;
    } else
      return k8[u];
  };
  // Global offset of copy u.  kLean: copies u and u + 2 of a wave cover rows
  // 16 apart (B not transposed: k-rows 4 apart), which the swizzles map to the
  // same chunks, so copies 2 and 3 add a uniform step to the offsets of 0 and
  // 1 at the copy (an opaque value, so that the sums are not hoisted out of
  // the main loop into registers of their own).  OOB_OFFSET plus a step stays
  // past every buffer range.
  const uint32_t a_step = 2u * C::A_ROWS_PER_DMA * (uint32_t)K * C::ES;
  const uint32_t b_step = BT ? a_step : 2u * C::B_ROWS_PER_DMA * (uint32_t)N * C::ES;
  static_assert(!kLean || (C::A_PW == 4 && C::B_PW == 4 && C::A_ROWS_PER_DMA == 8 && (BT || C::B_ROWS_PER_DMA == 2)),
                "the lean tile's copy offsets repeat every second copy");
  auto off_of = [&](const auto& off, int u, uint32_t step) -> uint32_t {
    if constexpr (kLean) {
      uint32_t v = off[u & 1];
      asm volatile("" : "+v"(v));
      return v + (uint32_t)(u >> 1) * step;
    } else {
      return off[u];
    }
  };
  auto issue_one = [&](const SlabSrd& r, int stage, int q) {
    if (q < C::A_PW) {
      dma16(r.a, copy_base() + C::a_buf(stage) + (wave * C::A_PW + q) * 1024u,
            r.kbase + k_of(a_k8, q, q) < (uint32_t)K ? off_of(a_off, q, a_step) : OOB_OFFSET);
    } else {
      const int u = q - C::A_PW;
      dma16(r.b, copy_base() + C::b_buf(stage) + (wave * C::B_PW + u) * 1024u,
            !BT || r.kbase + k_of(b_k8, u, q) < (uint32_t)K ? off_of(b_off, u, b_step) : OOB_OFFSET);
    }
  };

  // ------------------------------------------------------------------ fragments
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // 16-bit operands.  A fragment of block i, k-slice ks: row wm0 + 32i + lr,
  // logical chunk 2ks + lh.  a_swz depends on row bits 1..4 only, i.e. on lr:
  // block i adds 32 rows.
  uint32_t a_frag_off[C::NS];
#pragma unroll
  for (int ks = 0; ks < C::NS; ++ks)
    a_frag_off[ks] = (uint32_t)(wm0 + lr) * C::A_ROW + (((2u * ks + lh) ^ a_swz<C::A_CHUNKS>(lr)) << 4);
  // B fragment of block j, half t (k-slice 0; slice ks adds 16 k-rows, which
  // leaves b_swz unchanged): within 16-lane group g = lane/16 lane r = lane%16
  // addresses k-row 8(g/2) + 4t + r/4 and the 4 columns wn0 + 32j + 16(g%2) +
  // 4(r%4); the transposing read then gives lane l the k-values
  // 16ks + 8(l/32) + 4t .. +3 of column wn0 + 32j + l%32.
  const int g16 = lane >> 4, r16 = lane & 15;
  uint32_t b_frag_off[2][C::FN];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const uint32_t krow = 8 * (g16 >> 1) + 4 * t + (r16 >> 2);
      const uint32_t col = wn0 + 32 * j + 16 * (g16 & 1) + 4 * (r16 & 3);
      b_frag_off[t][j] = C::A_BYTES + krow * C::B_ROW + (((col >> 3) ^ b_swz<C::B_CHUNKS, C::ES>(krow)) << 4) +
                         (col & 4) * 2;
    }
  // fp8 operands.  A fragment of block i, k-slice ks (64 k-values): row
  // wm0 + 32i + lr, bytes 32 lh .. +31 of the slice, i.e. logical chunks
  // 4ks + 2lh and 4ks + 2lh + 1 (two 16-byte reads).
  uint32_t a8_off[C::NS][2];
#pragma unroll
  for (int ks = 0; ks < C::NS; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      a8_off[ks][h] = (uint32_t)(wm0 + lr) * C::A_ROW + (((4u * ks + 2u * lh + h) ^ a_swz<C::A_CHUNKS>(lr)) << 4);
  // B fragment of block j, k-slice 0, read q (0..3): within 16-lane group g
  // lane r addresses k-row 32(g/2) + 8q + r/2 and the 8 columns wn0 + 32j +
  // 16(g%2) + 8(r%2) .. +7; the 8-bit transposing read then gives lane l the
  // k-values 32(l/32) + 8q .. +7 of column wn0 + 32j + l%32.  The swizzle
  // depends on r/2 only, so read q adds 8q k-rows and slice ks 64ks.
  uint32_t b8_off[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const uint32_t krow = 32 * (g16 >> 1) + (r16 >> 1);
    const uint32_t col = wn0 + 32 * j + 16 * (g16 & 1) + 8 * (r16 & 1);
    b8_off[j] = C::A_BYTES + krow * C::B_ROW + (((col >> 4) ^ b_swz<C::B_CHUNKS, C::ES>(krow)) << 4) + (col & 8);
  }
  // Transposed B: fragment j is tile row wn0 + 32j + lr of the B tile, read
  // exactly like an A fragment (16-bit: logical chunk 2ks + lh; fp8: chunks
  // 4ks + 2lh and 4ks + 2lh + 1).
  uint32_t bt_off[C::NS][2];
#pragma unroll
  for (int ks = 0; ks < C::NS; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t chunk = C::ES == 2 ? 2u * ks + lh : 4u * ks + 2u * lh + h;
      bt_off[ks][h] = C::A_BYTES + (uint32_t)(wn0 + lr) * C::A_ROW + ((chunk ^ a_swz<C::A_CHUNKS>(lr)) << 4);
    }

  // 16x16 blocks (MI == 16), LDS offsets into buffer 0 of the operand;
  // another ring buffer, block or k-slice adds a constant that fits the LDS
  // read's 16-bit offset field.  A fragment of block i, k-slice ks (32 k-values): row
  // wm0 + 16i + l%16, k-values 32ks + 8(l/16) .. +7, i.e. logical chunk
  // 4ks + l/16 (a_swz depends on row bits 1..3 only, i.e. on l%16).  B
  // fragment of block j: within 16-lane group g = l/16 lane r = l%16 addresses
  // k-row 8g + 4t + r/4 (t = 0, 1: the two transposing reads) and the 4
  // columns wn0 + 16j + 4(r%4); the reads give lane l the k-values 8(l/16) ..
  // +7 of column wn0 + 16j + l%16, the operand layout of the 16x16x32 MFMA.
  // Transposed B: block j is tile row wn0 + 16j + l%16, read like A.
  constexpr bool M16 = C::MI == 16;
  const int lr16 = lane & 15;
  uint32_t a16_off[M16 ? C::NS : 1], bt16_off[M16 ? C::NS : 1], b16_off[M16 ? C::FN16 : 1];
  if constexpr (M16) {
    static_assert(BT || C::B_CHUNKS >= 8, "the 16x16 B swizzle covers rows of 128 bytes or more");
    // the largest constant a read adds: last ring buffer, k-slice and block
    static_assert((C::STAGES - 1) * C::A_BYTES + (C::FM16 - 1) * 16 * C::A_ROW + 16 * C::A_ROW < 65536 &&
                      (C::STAGES - 1) * C::B_BYTES +
                              (BT ? (C::FN16 - 1) * 16 * C::A_ROW : (32 * (C::NS - 1) + 4) * C::B_ROW) <
                          65536,
                  "a ring buffer's displacement must fit the LDS read offset");
#pragma unroll
    for (int ks = 0; ks < C::NS; ++ks) {
      const uint32_t chunk = ((4u * ks + (uint32_t)g16) ^ a_swz<C::A_CHUNKS>((uint32_t)lr16)) << 4;
      a16_off[ks] = C::a_buf(0) + (uint32_t)(wm0 + lr16) * C::A_ROW + chunk;
      bt16_off[ks] = C::b_buf(0) + (uint32_t)(wn0 + lr16) * C::A_ROW + chunk;
    }
#pragma unroll
    for (int j = 0; j < C::FN16; ++j) {
      const uint32_t krow = 8 * g16 + (r16 >> 2);
      const uint32_t col = wn0 + 16 * j + 4 * (r16 & 3);
      b16_off[j] = C::b_buf(0) + krow * C::B_ROW + (((col >> 3) ^ b_swz<C::B_CHUNKS, C::ES, C::MI>(krow)) << 4) +
                   (col & 4) * 2;
    }
  }

  // Per-buffer copies of the 16-bit fragment offsets, kept in registers: a
  // ring buffer lies STAGE_BYTES (64 KiB for the 256x256 tile) above the
  // previous one, beyond the 16-bit offset of an LDS read, so without them
  // every read address of a slab would be recomputed beside the MFMAs.  The
  // main loop runs whole turns of the ring, so the buffer index is a
  // compile-time constant.  (fp8 tiles keep the per-slab additions: there the
  // extra registers measured slower.)
  constexpr int S16 = C::ES == 2 && !M16 ? C::STAGES : 1;
  auto in_buffer = [](uint32_t off, int s) {
    uint32_t v = off + (uint32_t)(s * C::STAGE_BYTES);
    if (s > 0) asm volatile("" : "+v"(v));  // a register of its own, not re-derived in the loop
    return v;
  };
  uint32_t a_fo[S16][C::NS], b_fo[S16][2][C::FN], bt_fo[S16][C::NS];
  if constexpr (C::ES == 2 && !M16) {
#pragma unroll
    for (int s = 0; s < C::STAGES; ++s) {
#pragma unroll
      for (int ks = 0; ks < C::NS; ++ks) {
        a_fo[s][ks] = in_buffer(a_frag_off[ks], s);
        if constexpr (BT) bt_fo[s][ks] = in_buffer(bt_off[ks][0], s);
      }
      if constexpr (!BT) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          b_fo[s][0][j] = in_buffer(b_frag_off[0][j], s);
          b_fo[s][1][j] = in_buffer(b_frag_off[1][j], s);
        }
      }
    }
  }

  f32x16 acc[M16 ? 1 : C::FM][M16 ? 1 : C::FN];
#pragma unroll
  for (int i = 0; i < (M16 ? 1 : C::FM); ++i)
#pragma unroll
    for (int j = 0; j < (M16 ? 1 : C::FN); ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // 16x16 blocks: the main loop's accumulators (lane l: row 16i + l%16 of the
  // wave tile, columns 16j + 4(l/16) .. +3), moved into acc's 32x32 layout
  // after the loop
  f32x4 acc16[M16 ? C::FM16 : 1][M16 ? C::FN16 : 1];
#pragma unroll
  for (int i = 0; i < (M16 ? C::FM16 : 1); ++i)
#pragma unroll
    for (int j = 0; j < (M16 ? C::FN16 : 1); ++j) acc16[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Two fragment sets (k-slice being computed / k-slice being read).
  // 16-bit: A fragment i is one 16-byte read; B fragment j is two transposing
  // reads (lo: k 0..3, hi: k 4..7 of the lane's 8).  fp8: A fragment i is two
  // 16-byte reads, B fragment j four 8-bit transposing reads (k 8q .. 8q+7 of
  // the lane's 32).  A k-slice is read as NRD "pieces", in the order of first
  // use by the MFMAs (i outer, j inner): A0, then B0 .. B(FN-1), then A1 ..
  // A(FM-1).
  // (16x16 blocks: the same with FM16 x FN16 blocks of 16-byte A reads and
  // pairs of transposing B reads.)
  constexpr int FMB = M16 ? C::FM16 : C::FM, FNB = M16 ? C::FN16 : C::FN;  // fragments per k-slice
  constexpr int NMF = FMB * FNB;  // MFMAs per k-slice
  constexpr int RA = C::ES == 2 ? 1 : 2;                   // reads per A fragment
  constexpr int RB = BT ? RA : (C::ES == 2 ? 2 : 4);        // reads per B fragment
  constexpr int NRD = RA * FMB + RB * FNB;                  // LDS read instructions per k-slice
  u32x4 fa[kLean ? 1 : 2][FMB][RA];  // kLean: one set of A fragments (see lean_row)
  u32x2 fb[2][FNB][BT ? 1 : RB];
  u32x4 fbt[2][FNB][RA];  // transposed B: A-like 16-byte pieces
  auto read_piece = [&](int set, int stage, int ks, int piece) {
    if constexpr (M16) {
      if (piece < 1 || piece >= 1 + RB * FNB) {
        const int i = piece < 1 ? 0 : piece - RB * FNB;
        fa[kLean ? 0 : set][i][0] =
            *(const u32x4*)(smem + a16_off[ks] + (C::a_buf(stage) - C::a_buf(0)) + i * 16 * C::A_ROW);
      } else {
        const int j = (piece - 1) / RB, t = (piece - 1) % RB;
        constexpr uint32_t kB0 = C::b_buf(0);
        if constexpr (BT)
          fbt[set][j][0] =
              *(const u32x4*)(smem + bt16_off[ks] + (C::b_buf(stage) - kB0) + j * 16 * C::A_ROW);
        else
          fb[set][j][t] =
              lds_read_tr<DT>(smem + b16_off[j] + (C::b_buf(stage) - kB0) + (32 * ks + 4 * t) * C::B_ROW);
      }
    } else {
      const uint8_t* const st = smem + stage * C::STAGE_BYTES;
      if (piece < RA || piece >= RA + RB * C::FN) {
        const int t = piece < RA ? piece : piece - RB * C::FN;
        const int i = t / RA, h = t % RA;
        if constexpr (C::ES == 2)
          fa[set][i][0] = *(const u32x4*)(smem + a_fo[stage][ks] + i * 32 * C::A_ROW);
        else
          fa[set][i][h] = *(const u32x4*)(st + a8_off[ks][h] + i * 32 * C::A_ROW);
      } else {
        const int j = (piece - RA) / RB, t = (piece - RA) % RB;
        if constexpr (BT && C::ES == 2)
          fbt[set][j][t] = *(const u32x4*)(smem + bt_fo[stage][ks] + j * 32 * C::A_ROW);
        else if constexpr (BT)
          fbt[set][j][t] = *(const u32x4*)(st + bt_off[ks][t] + j * 32 * C::A_ROW);
        else if constexpr (C::ES == 2)
          fb[set][j][t] = lds_read_tr<DT>(smem + b_fo[stage][t][j] + ks * 16 * C::B_ROW);
        else
          fb[set][j][t] = lds_read_tr8(st + b8_off[j] + (ks * 64 + 8 * t) * C::B_ROW);
      }
    }
  };
  auto read_slice = [&](int set, int stage, int ks) {
#pragma unroll
    for (int q = 0; q < NRD; ++q) read_piece(set, stage, ks, q);
  };
  // MFMA t of a k-slice (i outer, j inner)
  auto mfma_one = [&](int set, int t) {
    if constexpr (M16) {
      const int i = t / C::FN16, j = t % C::FN16;
      const int sf = kLean ? 0 : set;
      if constexpr (BT)
        acc16[i][j] = mfma16<DT>(fbt[set][j][0], fa[sf][i][0], acc16[i][j]);
      else
        acc16[i][j] = mfma16<DT>(u32x4{fb[set][j][0][0], fb[set][j][0][1], fb[set][j][1][0], fb[set][j][1][1]},
                                 fa[sf][i][0], acc16[i][j]);
    } else {
      const int i = t / C::FN, j = t % C::FN;
      if constexpr (BT && C::ES == 2) {
        acc[i][j] = mfma32<DT>(fbt[set][j][0], fa[set][i][0], acc[i][j]);
      } else if constexpr (BT) {
        constexpr int FA = (F8 - 1) & 1, FB = (F8 - 1) >> 1;
        const u32x8 b8{fbt[set][j][0][0], fbt[set][j][0][1], fbt[set][j][0][2], fbt[set][j][0][3],
                       fbt[set][j][1][0], fbt[set][j][1][1], fbt[set][j][1][2], fbt[set][j][1][3]};
        const u32x8 a8{fa[set][i][0][0], fa[set][i][0][1], fa[set][i][0][2], fa[set][i][0][3],
                       fa[set][i][1][0], fa[set][i][1][1], fa[set][i][1][2], fa[set][i][1][3]};
        acc[i][j] = mfma32_f8<FB, FA>(b8, a8, acc[i][j]);
      } else if constexpr (C::ES == 2) {
        acc[i][j] = mfma32<DT>(u32x4{fb[set][j][0][0], fb[set][j][0][1], fb[set][j][1][0], fb[set][j][1][1]},
                               fa[set][i][0], acc[i][j]);
      } else {
        // B is the first operand (format FB), A the second (format FA)
        constexpr int FA = (F8 - 1) & 1, FB = (F8 - 1) >> 1;
        const u32x8 b8{fb[set][j][0][0], fb[set][j][0][1], fb[set][j][1][0], fb[set][j][1][1],
                       fb[set][j][2][0], fb[set][j][2][1], fb[set][j][3][0], fb[set][j][3][1]};
        const u32x8 a8{fa[set][i][0][0], fa[set][i][0][1], fa[set][i][0][2], fa[set][i][0][3],
                       fa[set][i][RA - 1][0], fa[set][i][RA - 1][1], fa[set][i][RA - 1][2], fa[set][i][RA - 1][3]};
        acc[i][j] = mfma32_f8<FB, FA>(b8, a8, acc[i][j]);
      }
    }
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int t = 0; t < NMF; ++t) mfma_one(set, t);
  };
  // Scheduling hint for one k-slice: alternate the MFMAs with the LDS reads
  // of the next k-slice, reads first, so neither the MFMA pipe nor the LDS
  // queue idles and the reads land well before the slice ends.
  constexpr int RD_PER_MF = (NRD + NMF - 1) / NMF;
  auto interleave = [&]() {
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   // one MFMA
      if (t * RD_PER_MF < NRD) __builtin_amdgcn_sched_group_barrier(0x100, RD_PER_MF, 0);  // LDS reads
    }
  };

  // kLean: the MFMAs of block row i of a k-slice (A fragment i, B fragments of
  // set `set`), then the reads of k-slice `rks` of ring buffer `rstage` that
  // this row frees or spreads: A fragment i (its last use was this row) and,
  // while any are left, one piece of the B fragments, into the other set.
  // The 16x16 blocks' accumulators go to the 32x32 layout in block_row.
  auto lean_row = [&](int set, int i, int rstage, int rks) {
#pragma unroll
    for (int j = 0; j < FNB; ++j) mfma_one(set, i * FNB + j);
    if (i < RB * FNB) read_piece(set ^ 1, rstage, rks, 1 + i);
    read_piece(set ^ 1, rstage, rks, i == 0 ? 0 : RB * FNB + i);
  };
  static_assert(!kLean || C::NS == 2, "lean 16x16 tile: two k-slices per slab");

  // ------------------------------------------------------------------ main loop
  // Ring of STAGES slabs; slab kt sits in buffer kt % STAGES.  Per slab:
  //   for each k-slice but the last: read the next k-slice | its MFMAs
  //   wait until this wave's reads of the slab returned and its loads of slab
  //     kt+1 landed; barrier (slab kt+1 is complete for every wave, and no
  //     wave reads this buffer any more)
  //   refill this buffer with slab kt+STAGES; read k-slice 0 of slab kt+1 |
  //     MFMAs of the last k-slice
  // Set parity: k-slice ks of a slab computes from set ks % 2; BK/16 is even,
  // so the next slab's first slice lands in set 0.
  static_assert(C::NS % 2 == 0, "the fragment sets alternate per k-slice");
  if (KT > 0) {
#pragma unroll
    for (int s = 0; s < C::STAGES; ++s) {
      const SlabSrd r = slab_srd(s);
#pragma unroll
      for (int q = 0; q < C::PW; ++q) issue_one(r, s, q);
    }
    wait_vmcnt<(C::STAGES - 1) * C::PW>();
    __syncthreads();
    read_slice(0, 0, 0);
    // slab kt sits in ring buffer st = kt % STAGES (a constant in each copy
    // of the body below)
    // refill == false (the slabs after the loop; fp8 tiles of two waves per SIMD): the
    // slab kt + STAGES that would be loaded lies past K, and with a two-slab
    // ring the wait above is for every load anyway, so no empty loads need
    // to keep the count
    auto slab = [&](int kt, int st, bool refill) {
      const int st_next = st + 1 == C::STAGES ? 0 : st + 1;
      if constexpr (kLean) {
        // k-slice 0 (set 0), reading k-slice 1 of this slab
#pragma unroll
        for (int i = 0; i < FMB; ++i) lean_row(0, i, st, 1);
      } else {
#pragma unroll
        for (int ks = 0; ks < C::NS - 1; ++ks) {
          read_slice((ks + 1) & 1, st, ks + 1);
          mfmas(ks & 1);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lgkmcnt<0>();
      wait_vmcnt<(C::STAGES - 2) * C::PW>();
      // a bare s_barrier: the copies it publishes were waited for above
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const SlabSrd r = slab_srd(kt + C::STAGES);
      if constexpr (kTight) {
        // fp8, two waves per SIMD: the refill is spread over the last
        // k-slice, in program order MFMA t, then its share of the next
        // slab's first-slice reads, then its share of this wave's copies
        // (one per MFMA).  Issued in one burst after the MFMAs, the copies
        // of all eight waves kept the address unit's command queue full
        // (SQ_VMEM_TA_CMD_FIFO_FULL) and stalled the waves behind them:
        // spread, 8192^3 E4M3 runs 4-5 % faster.  Every copy takes the k
        // check here: a uniform branch around copies inside the MFMA
        // sequence made the compiler spill.
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
          mfma_one((C::NS - 1) & 1, t);
#pragma unroll
          for (int pc = t * NRD / NMF; pc < (t + 1) * NRD / NMF; ++pc) read_piece(0, st_next, 0, pc);
          if (refill) {
#pragma unroll
            for (int q = t * C::PW / NMF; q < (t + 1) * C::PW / NMF; ++q) issue_one(r, st, q);
          }
        }
      } else if constexpr (C::NW == 8) {
        // two waves per SIMD, 16-bit tiles: the A refill goes out right
        // after the barrier, the last k-slice's reads and MFMAs next, the B
        // refill after them (measured 1.5-2 % faster on the large shapes than
        // the whole refill after the MFMAs, which is faster than the whole
        // refill first; spreading the copies one per MFMA as the fp8 tile
        // does was 2-4 % slower here).  A uniform branch drops the per-lane
        // k check of the A copies in every slab below K.
        const uint32_t sa = (kLean ? copy_base() : smem_lds) + C::a_buf(st);
        if (!kLean || refill) {
          if (r.full) {
#pragma unroll
            for (int q = 0; q < C::A_PW; ++q) dma16(r.a, sa + (wave * C::A_PW + q) * 1024u, off_of(a_off, q, a_step));
          } else {
#pragma unroll
            for (int q = 0; q < C::A_PW; ++q) issue_one(r, st, q);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kLean) {
          // k-slice 1 (set 1), reading k-slice 0 of the next slab
#pragma unroll
          for (int i = 0; i < FMB; ++i) lean_row(1, i, st_next, 0);
        } else {
          read_slice(0, st_next, 0);
          mfmas((C::NS - 1) & 1);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
        if (!kLean || refill) {
#pragma unroll
          for (int q = C::A_PW; q < C::PW; ++q) issue_one(r, st, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // one wave per SIMD: the refill loads go out one at a time between the
        // reads of the next k-slice (and so between the MFMAs), never as a
        // burst that would back up the address unit and stall MFMA issue
        // (64x64 tiles: in slabs below K the A copies skip their per-lane k
        // check; measured 4 % faster there, and no faster for 128x128)
        if (C::BM * C::BN <= 64 * 64 && r.full) {
          const uint32_t sa = copy_base() + C::a_buf(st);
#pragma unroll
          for (int q = 0; q < C::PW; ++q) {
            if (q < C::A_PW)
              dma16(r.a, sa + (wave * C::A_PW + q) * 1024u, a_off[q]);
            else
              issue_one(r, st, q);
#pragma unroll
            for (int pc = q * NRD / C::PW; pc < (q + 1) * NRD / C::PW; ++pc) read_piece(0, st_next, 0, pc);
          }
        } else {
#pragma unroll
          for (int q = 0; q < C::PW; ++q) {
            issue_one(r, st, q);
#pragma unroll
            for (int pc = q * NRD / C::PW; pc < (q + 1) * NRD / C::PW; ++pc) read_piece(0, st_next, 0, pc);
          }
        }
        mfmas((C::NS - 1) & 1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int kt = 0;
    for (; kt + C::STAGES <= KT; kt += C::STAGES) {
#pragma unroll
      for (int s = 0; s < C::STAGES; ++s) slab(kt + s, s, true);
    }
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
      if (kt + s < KT) slab(kt + s, s, !((kTight || kLean) && C::STAGES == 2));
  }

  // The epilogue takes the accumulators one 32-row block-row at a time, in
  // the 32x32 layout.  16x16 blocks are moved into it there, so that only one
  // block-row's converted values are live: region (I, J) of 32 x 32 holds
  // blocks (2I + r, 2J + c).  For fixed c and register e, the value of block
  // row r that lane (s, bit4 = h, bit5 = t) holds (row 16r + s, column
  // 16c + 8t + 4h + e) belongs to lane (s, bit4 = r, bit5 = h), at register
  // 4(2c + t) + e (row s + 16r, column 8(2c + t) + 4h + e): the three bits
  // (register r, lane bit 4, lane bit 5) rotate, which is a swap of the
  // register with lane bit 4 (v_permlane16_swap) followed by a swap with lane
  // bit 5 (v_permlane32_swap).
  auto block_row = [&](int I, f32x16 (&row)[C::FN]) {
    if constexpr (M16) {
#pragma unroll
      for (int J = 0; J < C::FN; ++J)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = acc16[2 * I][2 * J + c][e], y = acc16[2 * I + 1][2 * J + c][e];
            swap16(x, y);
            swap32(x, y);
            row[J][4 * (2 * c) + e] = x;
            row[J][4 * (2 * c + 1) + e] = y;
          }
    } else {
#pragma unroll
      for (int J = 0; J < C::FN; ++J) row[J] = acc[I][J];
    }
  };

  // fp8: the product of the two per-tensor scales (uniform; NULL reads as 1),
  // loaded only now so that no register holds it through the main loop
  float scale = 1.0f;
  if constexpr (F8 != 0) {
    const float sa = p.scale_a != nullptr ? *p.scale_a : 1.0f;
    const float sb = p.scale_b != nullptr ? *p.scale_b : 1.0f;
    scale = sa * sb;
  }
  // drain: no load may still be writing LDS when the workgroup retires
  wait_vmcnt<0>();
  // the ring is free once every wave is past its last fragment read
  __syncthreads();
  epilogue_store<DT, EPI, C::WM, C::WN, F8 != 0, C::FM, C::FN>(p, block_row, m0, n0, wm0, wn0, kTight || kLean ? lane_fresh() : lane,
                                                               smem + wave * C::EPI_STAGE, bias_lds,
                                                               (float*)(smem + C::RED_OFF), scale);
}

}  // namespace egm
