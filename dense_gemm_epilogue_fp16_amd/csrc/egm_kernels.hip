// egm_kernels.hip - instantiates the fused GEMM + epilogue kernel for every
// (epilogue, tile config) and the stand-alone epilogue kernels for one dtype.
// Built once per 16-bit dtype (-DEGM_DTYPE=0 fp16, 1 bf16) and, with
// -DEGM_F8=1..4, once per (fp8 format pair, 16-bit output dtype): the forward
// epilogues only, on one-byte tiles with 128-deep k-slabs (the same bytes per
// slab row as the 64-deep 16-bit slabs).
#include <utility>

#include "egm_epilogue.hpp"
#include "egm_gemm.hpp"
#include "egm_launch.hpp"
#include "egm_layernorm.hpp"

#ifndef EGM_DTYPE
#error "EGM_DTYPE must be 0 (fp16) or 1 (bf16)"
#endif
#ifndef EGM_F8
#define EGM_F8 0
#endif
// -DEGM_LEAN=1 / 2: only the lean tile's kernels (config 7), for B not
// transposed with the forward epilogues (1) or for the rest (2), each unit
// compiled with the instruction scheduler that keeps its kernels free of
// scratch and fastest (build.py); every other unit leaves them out
#ifndef EGM_LEAN
#define EGM_LEAN 0
#endif
#if EGM_LEAN && EGM_F8
#error "the lean tile is built for 16-bit operands only"
#endif

namespace egm {
namespace {

constexpr int DT = EGM_DTYPE;
constexpr int F8 = EGM_F8;
constexpr int ES = F8 == 0 ? 2 : 1;

template <int EPI, int CFG, bool BT>
void launch_gemm(dim3 grid, hipStream_t s, const GemmArgs& a) {
  constexpr ConfigInfo ci = kConfigs[CFG];
  using C = TileCfg<ci.bm, ci.bn, ci.stages, ci.wm, ci.wn, ci.bk * (2 / ES), ES, ci.mi>;
  hipLaunchKernelGGL((gemm_epilogue_kernel<DT, EPI, C, F8, BT>), grid, dim3(C::NT), 0, s, a);
}

// configs this unit builds: 16x16 MFMA blocks are 16-bit only, and the lean
// tile lives in units of its own
template <int CFG>
constexpr bool built_here() {
  return (F8 == 0 || kConfigs[CFG].mi == 32) && lean_config(CFG) == (EGM_LEAN != 0);
}

// a config this unit builds, named in place of those it does not (the
// conditional below instantiates both of its branches)
constexpr int fallback_config() {
  for (int c = 0; c < kNumConfigs; ++c)
    if (lean_config(c) == (EGM_LEAN != 0)) return c;
  return 0;
}

template <int EPI, bool BT, int... CFG>
GemmLaunch pick_gemm(int cfg, std::integer_sequence<int, CFG...>) {
  GemmLaunch out = nullptr;
  ((cfg == CFG ? (out = built_here<CFG>() ? &launch_gemm<EPI, (built_here<CFG>() ? CFG : fallback_config()), BT>
                                          : nullptr)
               : out),
   ...);
  return out;
}

#if EGM_F8 == 0 && !EGM_LEAN
template <int EPI>
void launch_epi(dim3 grid, hipStream_t s, const EpiArgs& a) {
  hipLaunchKernelGGL((epilogue_kernel<DT, EPI>), grid, dim3(256), 0, s, a);
}

void launch_partials(dim3 grid, hipStream_t s, const void* D, int64_t M, int32_t N, int32_t layout, float* partial) {
  hipLaunchKernelGGL((axis_partials_kernel<DT>), grid, dim3(256), 0, s, D, M, N, layout, partial);
}

template <int CFG, bool RES>
void launch_ln(dim3 grid, hipStream_t s, const LnArgs& a) {
  constexpr LnConfig c = kLnConfigs[CFG];
  hipLaunchKernelGGL((layernorm_kernel<DT, c.tpr, c.cpt, RES>), grid, dim3(256), 0, s, a);
}

template <bool RES>
LnLaunch ln_row(int cfg) {
  static_assert(kNumLnConfigs == 7, "update the LayerNorm launch table with its config table");
  switch (cfg) {
    case 0: return &launch_ln<0, RES>;
    case 1: return &launch_ln<1, RES>;
    case 2: return &launch_ln<2, RES>;
    case 3: return &launch_ln<3, RES>;
    case 4: return &launch_ln<4, RES>;
    case 5: return &launch_ln<5, RES>;
    case 6: return &launch_ln<6, RES>;
    default: return nullptr;
  }
}
#endif

// the (epilogue, B layout) pairs this unit builds
template <int EPI, bool BT>
constexpr bool unit_builds() {
  return EGM_LEAN == 0 || lean_unit(EPI, BT) == EGM_LEAN;
}

template <int EPI, bool BT>
GemmLaunch gemm_row(int cfg) {
  if constexpr (unit_builds<EPI, BT>())
    return pick_gemm<EPI, BT>(cfg, std::make_integer_sequence<int, kNumConfigs>{});
  else
    return nullptr;
}

template <bool BT>
GemmLaunch gemm_table_bt(int epi, int cfg) {
  switch (epi) {
    case EPI_NONE: return gemm_row<EPI_NONE, BT>(cfg);
    case EPI_BIAS: return gemm_row<EPI_BIAS, BT>(cfg);
    case EPI_RELU: return gemm_row<EPI_RELU, BT>(cfg);
    case EPI_GELU: return gemm_row<EPI_GELU, BT>(cfg);
    case EPI_RELU_AUX: return gemm_row<EPI_RELU_AUX, BT>(cfg);
    case EPI_RESID: return gemm_row<EPI_RESID, BT>(cfg);
#if EGM_F8 == 0
    case EPI_DRELU: return gemm_row<EPI_DRELU, BT>(cfg);
    case EPI_DRELU_BGRAD: return gemm_row<EPI_DRELU_BGRAD, BT>(cfg);
#endif
    default: return nullptr;
  }
}

GemmLaunch gemm_table(int epi, int cfg, bool bt) { return bt ? gemm_table_bt<true>(epi, cfg) : gemm_table_bt<false>(epi, cfg); }

#if EGM_F8 == 0 && !EGM_LEAN
EpiLaunch epi_table(int epi) {
  switch (epi) {
    case EPI_BIAS: return &launch_epi<EPI_BIAS>;
    case EPI_RELU: return &launch_epi<EPI_RELU>;
    case EPI_GELU: return &launch_epi<EPI_GELU>;
    case EPI_RELU_AUX: return &launch_epi<EPI_RELU_AUX>;
    case EPI_RESID: return &launch_epi<EPI_RESID>;
    case EPI_DRELU: return &launch_epi<EPI_DRELU>;
    default: return nullptr;
  }
}
#endif

}  // namespace

#if EGM_LEAN == 1 && EGM_DTYPE == 0
GemmLaunch gemm_launcher_lean1_f16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
#elif EGM_LEAN == 1
GemmLaunch gemm_launcher_lean1_bf16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
#elif EGM_LEAN == 2 && EGM_DTYPE == 0
GemmLaunch gemm_launcher_lean2_f16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
#elif EGM_LEAN == 2
GemmLaunch gemm_launcher_lean2_bf16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
#elif EGM_F8 != 0
#define EGM_CAT3(a, b, c) a##b##_##c
#define EGM_FP8_LAUNCHER(dt, f8) EGM_CAT3(gemm_launcher_fp8_, dt, f8)
GemmLaunch EGM_FP8_LAUNCHER(EGM_DTYPE, EGM_F8)(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
#elif EGM_DTYPE == 0
LnLaunch layernorm_launcher_f16(int cfg, bool residual) { return residual ? ln_row<true>(cfg) : ln_row<false>(cfg); }
GemmLaunch gemm_launcher_f16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
EpiLaunch epi_launcher_f16(int epi) { return epi_table(epi); }
PartialsLaunch partials_launcher_f16() { return &launch_partials; }
void launch_bias_grad_finish(dim3 grid, hipStream_t s, const float* partial, int64_t chunks, int64_t len,
                             float* out) {
  hipLaunchKernelGGL(bias_grad_finish_kernel<float>, grid, dim3(256), 0, s, partial, chunks, len, out);
}
#else
LnLaunch layernorm_launcher_bf16(int cfg, bool residual) { return residual ? ln_row<true>(cfg) : ln_row<false>(cfg); }
GemmLaunch gemm_launcher_bf16(int epi, int cfg, bool bt) { return gemm_table(epi, cfg, bt); }
EpiLaunch epi_launcher_bf16(int epi) { return epi_table(epi); }
PartialsLaunch partials_launcher_bf16() { return &launch_partials; }
#endif

}  // namespace egm
