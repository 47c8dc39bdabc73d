// egm_launch.hpp - the table of tile configurations and the launch entry
// points that the per-dtype kernel translation units provide to the host API.
#pragma once

#include <hip/hip_runtime.h>

#include "egm_device.hpp"

namespace egm {

struct GemmArgs;
struct EpiArgs;

struct ConfigInfo {
  int bm, bn;      // output tile
  int wm, wn;      // waves along m and n (the workgroup is 64 * wm * wn lanes)
  int stages;      // LDS ring depth, in 32-deep k-slabs
  double rel_eff;  // relative per-CU MFMA efficiency, used by the shape heuristic
};

// Tile configurations: 32x32x16 MFMA blocks, 32-deep k-slabs.  The 256x256
// tile runs 8 waves (2 per SIMD, 64x128 each) so that one wave's MFMAs can
// issue while its SIMD partner waits on LDS reads or copies; the smaller tiles
// run 4 waves (2 x 2).
inline constexpr ConfigInfo kConfigs[] = {
    {256, 256, 4, 2, 4, 1.00},
    {256, 128, 2, 2, 4, 0.90},
    {128, 256, 2, 2, 4, 0.90},
    {128, 128, 2, 2, 4, 0.75},
    {64, 64, 2, 2, 4, 0.40},
};
inline constexpr int kNumConfigs = int(sizeof(kConfigs) / sizeof(kConfigs[0]));

using GemmLaunch = void (*)(dim3 grid, hipStream_t stream, const GemmArgs& args);
using EpiLaunch = void (*)(dim3 grid, hipStream_t stream, const EpiArgs& args);

// Defined in egm_kernels.hip (compiled once per dtype).
GemmLaunch gemm_launcher_f16(int epi, int cfg);
GemmLaunch gemm_launcher_bf16(int epi, int cfg);
EpiLaunch epi_launcher_f16(int epi);
EpiLaunch epi_launcher_bf16(int epi);

inline GemmLaunch gemm_launcher(int dt, int epi, int cfg) {
  return dt == DT_F16 ? gemm_launcher_f16(epi, cfg) : gemm_launcher_bf16(epi, cfg);
}
inline EpiLaunch epi_launcher(int dt, int epi) { return dt == DT_F16 ? epi_launcher_f16(epi) : epi_launcher_bf16(epi); }

}  // namespace egm
