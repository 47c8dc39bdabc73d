// egm_launch.hpp - the table of tile configurations and the launch entry
// points that the per-dtype kernel translation units provide to the host API.
#pragma once

#include <hip/hip_runtime.h>

#include "egm_device.hpp"

namespace egm {

struct GemmArgs;
struct EpiArgs;
struct LnArgs;

// LayerNorm row kernel shapes: tpr threads per row (64: one wave; 256: a
// workgroup), each holding cpt 16-byte chunks; rows up to tpr * cpt * 8
// elements.  The host picks the first config whose capacity covers the row.
struct LnConfig {
  int tpr, cpt;
};
inline constexpr LnConfig kLnConfigs[] = {{64, 1}, {64, 2}, {64, 4}, {64, 8}, {256, 4}, {256, 8}, {256, 16}};
inline constexpr int kNumLnConfigs = int(sizeof(kLnConfigs) / sizeof(kLnConfigs[0]));
using LnLaunch = void (*)(dim3 grid, hipStream_t stream, const LnArgs& args);
LnLaunch layernorm_launcher_f16(int cfg, bool residual);
LnLaunch layernorm_launcher_bf16(int cfg, bool residual);

struct ConfigInfo {
  int bm, bn;      // output tile
  int wm, wn;      // waves along m and n (the workgroup is 64 * wm * wn lanes)
  int stages;      // LDS ring depth, in k-slabs
  int bk;          // k-slab depth (32 or 64)
  double rel_eff;  // relative per-CU MFMA efficiency, used by the shape heuristic
  int mi;          // MFMA block: 32 (32x32x16) or 16 (16x16x32; 16-bit operands only)
};

// Tile configurations: 64-deep k-slabs (128-byte A rows: whole cache lines
// per row, half the barriers of 32-deep slabs).  The 256x256 tile runs 8
// waves (2 per SIMD, 2 x 4 of 128x64 each) so that one wave's MFMAs can issue
// while its SIMD partner waits on LDS reads or copies; its 64 KiB slabs leave
// room for a ring of 2.  The smaller tiles run 4 waves (2 x 2) with deeper rings.
// 32x32x16 MFMA blocks, except configs 5-7, with 16x16x32 blocks (16-bit
// operands only): config 5, the 64x64 tile (four independent accumulator
// chains per 32x32 wave tile instead of one), which the per-shape choice
// takes over config 4; config 6, the 32x64 tile of two waves; and config 7,
// the 256x256 tile of config 0 with 16x16x32 blocks and one set of
// fragments (the "lean" tile: 16x16x32 MFMAs sustain more flops than
// 32x32x16 ones at the board's power limit, and only a single fragment set
// fits beside the accumulators at two waves per SIMD).  Config 7's kernels
// are compiled in units of their own with other instruction schedulers (see
// build.py); the per-shape choice takes it over config 0 for 16-bit
// operands where it measured faster: from K = 2048 on for the kernels with B
// not transposed and no mask, from K = kLeanMinK on for the others.
inline constexpr ConfigInfo kConfigs[] = {
    {256, 256, 2, 4, 2, 64, 1.00, 32},
    {256, 128, 2, 2, 3, 64, 0.90, 32},
    {128, 256, 2, 2, 3, 64, 0.90, 32},
    {128, 128, 2, 2, 4, 64, 0.75, 32},
    {64, 64, 2, 2, 4, 64, 0.40, 32},
    {64, 64, 2, 2, 4, 64, 0.41, 16},
    {32, 64, 1, 2, 4, 64, 0.25, 16},
    {256, 256, 2, 4, 2, 64, 1.02, 16},
};
inline constexpr int kNumConfigs = int(sizeof(kConfigs) / sizeof(kConfigs[0]));
// the lean tile: 16x16x32 blocks with 8 waves (built in its own units)
constexpr bool lean_config(int c) { return kConfigs[c].mi == 16 && kConfigs[c].wm * kConfigs[c].wn == 8; }
// the shortest K for which the per-shape choice considers the lean tile for
// every kernel (those with B not transposed and no mask: from K = 2048 on)
inline constexpr int64_t kLeanMinK = 12288;

using GemmLaunch = void (*)(dim3 grid, hipStream_t stream, const GemmArgs& args);
using EpiLaunch = void (*)(dim3 grid, hipStream_t stream, const EpiArgs& args);
// bias gradient of the two-kernel path: partial sums of D (see axis_partials_kernel)
using PartialsLaunch = void (*)(dim3 grid, hipStream_t stream, const void* D, int64_t M, int32_t N,
                                int32_t layout, float* partial);

// Defined in egm_kernels.hip (compiled once per dtype).
// bt: B given transposed ([N, K] row-major)
GemmLaunch gemm_launcher_f16(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_bf16(int epi, int cfg, bool bt);
// the lean tile's kernels (egm_kernels.hip built with -DEGM_LEAN=1: B not
// transposed, forward epilogues; -DEGM_LEAN=2: the others)
GemmLaunch gemm_launcher_lean1_f16(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_lean1_bf16(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_lean2_f16(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_lean2_bf16(int epi, int cfg, bool bt);
// which lean unit builds an (epilogue, B layout): 1 or 2
constexpr int lean_unit(int epi, bool bt) { return !bt && !epi_reads_mask(epi) ? 1 : 2; }
EpiLaunch epi_launcher_f16(int epi);
EpiLaunch epi_launcher_bf16(int epi);
PartialsLaunch partials_launcher_f16();
PartialsLaunch partials_launcher_bf16();
// the last step of every bias gradient (dtype-independent; in the fp16 unit)
void launch_bias_grad_finish(dim3 grid, hipStream_t stream, const float* partial, int64_t chunks, int64_t len,
                             float* out);

// fp8 operands (defined in egm_kernels.hip built with -DEGM_F8): one table per
// (output dtype 0 fp16 / 1 bf16, format pair f8 = 1 + fa + 2 fb); forward
// epilogues only (nullptr otherwise)
GemmLaunch gemm_launcher_fp8_0_1(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_0_2(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_0_3(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_0_4(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_1_1(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_1_2(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_1_3(int epi, int cfg, bool bt);
GemmLaunch gemm_launcher_fp8_1_4(int epi, int cfg, bool bt);

inline GemmLaunch gemm_launcher_fp8(int dt, int f8, int epi, int cfg, bool bt) {
  using Table = GemmLaunch (*)(int, int, bool);
  static constexpr Table tables[2][4] = {
      {&gemm_launcher_fp8_0_1, &gemm_launcher_fp8_0_2, &gemm_launcher_fp8_0_3, &gemm_launcher_fp8_0_4},
      {&gemm_launcher_fp8_1_1, &gemm_launcher_fp8_1_2, &gemm_launcher_fp8_1_3, &gemm_launcher_fp8_1_4}};
  if ((dt != DT_F16 && dt != DT_BF16) || f8 < 1 || f8 > 4) return nullptr;
  return tables[dt == DT_F16 ? 0 : 1][f8 - 1](epi, cfg, bt);
}

inline GemmLaunch gemm_launcher(int dt, int epi, int cfg, bool bt) {
  if (cfg >= 0 && cfg < kNumConfigs && lean_config(cfg)) {
    if (lean_unit(epi, bt) == 1)
      return dt == DT_F16 ? gemm_launcher_lean1_f16(epi, cfg, bt) : gemm_launcher_lean1_bf16(epi, cfg, bt);
    return dt == DT_F16 ? gemm_launcher_lean2_f16(epi, cfg, bt) : gemm_launcher_lean2_bf16(epi, cfg, bt);
  }
  return dt == DT_F16 ? gemm_launcher_f16(epi, cfg, bt) : gemm_launcher_bf16(epi, cfg, bt);
}
inline EpiLaunch epi_launcher(int dt, int epi) { return dt == DT_F16 ? epi_launcher_f16(epi) : epi_launcher_bf16(epi); }
inline PartialsLaunch partials_launcher(int dt) { return dt == DT_F16 ? partials_launcher_f16() : partials_launcher_bf16(); }

}  // namespace egm
