// egm_api.hip - host side of the C ABI declared in include/egm.h: argument
// validation, per-shape tile-config choice, optional autotune, and the
// launches of the fused kernel or of the two-kernel measurement path.
//
// Pages (cited by title):
//   [bias-fusion] "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
//                 body: plan(epilog, epilog_inputs) / execute / free; the
//                 checklist (matching dtypes; bias (m,1) or (1,n), anything
//                 else fails; free releases the plan; autotune via options).
//   [bindings]    "nvmath-python：cuBLAS与cuSOLVER的Python绑定加速ML线性代数"
//                 body, checklist items 2-3: plan() picks the algorithm,
//                 execute() is asynchronous on a stream, the choice is logged.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <unordered_map>

#include "egm.h"
#include "egm_epilogue.hpp"
#include "egm_gemm.hpp"
#include "egm_launch.hpp"
#include "egm_layernorm.hpp"

namespace {

using egm::EpiArgs;
using egm::EpiLaunch;
using egm::GemmArgs;
using egm::GemmLaunch;

constexpr int kNumEpi = 8;
// keeps every in-tile buffer offset (256 rows x n or k elements) below 2^30
constexpr int64_t kMaxNK = int64_t(1) << 21;
constexpr int kNumCUs = 256;

using egm::kConfigs;
using egm::kNumConfigs;
using egm::ConfigInfo;

// egm_epilog_t -> device epilogue kind (the enum values coincide by design)
int epi_of(egm_epilog_t e) { return int(e); }

const char* epilog_name(int e) {
  static const char* names[kNumEpi] = {"DEFAULT",       "BIAS",          "RELU_BIAS", "GELU_BIAS",
                                       "RELU_AUX_BIAS", "BIAS_RESIDUAL", "DRELU",     "DRELU_BGRAD"};
  return (e >= 0 && e < kNumEpi) ? names[e] : "?";
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A launch of config c is one workgroup per output tile along grid.x, and a
// grid dimension holds at most 2^32 - 1 work-items (workgroups x threads).
bool grid_fits(int64_t m, int64_t n, int c) {
  const int64_t tiles = cdiv(m, kConfigs[c].bm) * cdiv(n, kConfigs[c].bn);
  return tiles * 64 * kConfigs[c].wm * kConfigs[c].wn <= int64_t(0xffffffff);
}

// Configs built for the operand type: 16x16 MFMA blocks exist for 16-bit
// operands only.
bool config_built(int c, bool fp8) { return !fp8 || kConfigs[c].mi == 32; }

// The shortest K for which the per-shape choice considers the lean tile for
// a GEMM kernel with B not transposed whose epilogue neither writes nor reads
// the ReLU mask (every other kernel: kLeanMinK).
constexpr int64_t kLeanMinKPlain = 2048;
bool lean_plain(int gemm_epi, bool bt) {
  return egm::lean_unit(gemm_epi, bt) == 1 && gemm_epi != egm::EPI_RELU_AUX;
}

// The per-shape choice takes the lean 256x256 tile (16x16x32 blocks) only
// where it measured faster than config 0.  Kernels with B not transposed and
// no mask: 0.5-5 % faster from K = 2048 on (8192x8192x2048 to 8192^3, bf16
// and fp16, the bias, ReLU, GELU and residual epilogues; 4096^3 GELU 5 %;
// 2.5-5.3 % on the 17 shapes of an 87-shape fp16 sweep where it is chosen),
// equal at K = 1024 (the FFN up-projection), mostly 2-4 % slower at K = 512.
// The others (the mask epilogue, B transposed, the backward epilogues): from
// K = 16384 on equal (the mask) to 3.5 % faster (B transposed), at K = 8192
// 1-4 % slower.  gemm_epi: the epilogue the GEMM kernel itself applies
// (EPI_NONE on the two-kernel path).
bool config_considered(int c, bool fp8, int64_t k, int gemm_epi, bool bt) {
  if (!config_built(c, fp8)) return false;
  if (!egm::lean_config(c)) return true;
  return k >= (lean_plain(gemm_epi, bt) ? kLeanMinKPlain : egm::kLeanMinK);
}

// Per-shape choice: among the configs whose grid fits, the one with the
// smallest estimated time, counting whole waves of tiles over the 256 CUs,
// scaled by the config's relative efficiency.  Ties go to the lower id.  -1
// when no config fits.  gemm_epi, bt: the GEMM kernel's epilogue and B
// layout (config_considered).  batch > 1: a strided batch of that many
// problems in one launch (grid.y), whose tiles fill the CUs together.
int choose_config(int64_t m, int64_t n, int64_t k, bool fp8, int gemm_epi, bool bt, int64_t batch = 1) {
  int best = -1;
  double best_t = 0;
  for (int c = 0; c < kNumConfigs; ++c) {
    if (!grid_fits(m, n, c) || !config_considered(c, fp8, k, gemm_epi, bt)) continue;
    const int64_t tiles = cdiv(m, kConfigs[c].bm) * cdiv(n, kConfigs[c].bn) * batch;
    const int64_t waves = cdiv(tiles, kNumCUs);
    const double t = double(waves) * kConfigs[c].bm * kConfigs[c].bn * double(k > 0 ? k : 1) / kConfigs[c].rel_eff;
    if (best < 0 || t < best_t * 0.999) {
      best = c;
      best_t = t;
    }
  }
  return best;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct egm_plan_s {
  int64_t m, n, k;
  egm_dtype_t dtype;
  egm_epilog_t epilog;
  const void* bias;
  int32_t bias_layout;
  const void* residual;
  void* bias_grad;           // DRELU_BGRAD output (fp32)
  int32_t fused;
  std::atomic<int32_t> config;            // rewritten once by a pending autotune
  int32_t group_m;
  int32_t chosen_per_shape;               // config from the per-shape choice (not forced, not autotuned)
  std::atomic<int32_t> autotune_pending;
  std::mutex tune_mu;                     // one autotune per plan, even from several threads
  size_t workspace_bytes;
  size_t product_bytes;      // the two-kernel path's P at the start of the workspace
  int64_t grad_len;          // DRELU_BGRAD: length of the gradient (n or m)
  int32_t f8;                // 0: 16-bit operands; 1 + fa + 2 fb: fp8 operands (formats of A, B)
  const float* scale_a;      // fp8: per-tensor scales (device, may be NULL)
  const float* scale_b;
  int32_t b_transposed;      // B given as [N, K] row-major
};

namespace {

// The epilogue the GEMM kernel applies: the plan's, or none on the
// two-kernel path (where a second kernel applies it).
int gemm_epi_of(const egm_plan_s* p) {
  const int epi = epi_of(p->epilog);
  return !p->fused && epi != egm::EPI_NONE ? int(egm::EPI_NONE) : epi;
}

// Live plans.  A handle is a number handed out once and never again, not the
// plan's address: a NULL, freed or foreign handle is recognised by a lookup
// that never touches freed memory, and a stale handle cannot alias a later
// plan.  Each call holds a reference for its duration, so an egm_free of the
// same handle from another thread cannot release the plan under it.
struct Registry {
  std::mutex mu;
  std::unordered_map<uintptr_t, std::shared_ptr<egm_plan_s>> live;
  uintptr_t next = 0x1000;  // handles start well away from NULL
};
Registry& registry() {
  static Registry* r = new Registry();  // never destroyed: usable from exit handlers
  return *r;
}

egm_plan_t register_plan(std::shared_ptr<egm_plan_s> p) {
  Registry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  const uintptr_t h = r.next;
  r.live.emplace(h, std::move(p));
  r.next += 0x10;
  return reinterpret_cast<egm_plan_t>(h);
}

std::shared_ptr<egm_plan_s> lookup(egm_plan_t handle) {
  if (handle == nullptr) return nullptr;
  Registry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  const auto it = r.live.find(reinterpret_cast<uintptr_t>(handle));
  return it == r.live.end() ? nullptr : it->second;
}

// removes the handle; the plan itself goes when the last call using it returns
bool unregister(egm_plan_t handle) {
  std::shared_ptr<egm_plan_s> dead;  // released after the lock
  Registry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  const auto it = r.live.find(reinterpret_cast<uintptr_t>(handle));
  if (it == r.live.end()) return false;
  dead = std::move(it->second);
  r.live.erase(it);
  return true;
}

// DRELU_BGRAD partial-sum rows a launch writes: one per tile row ((1,n)
// bias) or tile column ((m,1) bias) on the fused path, one per 32-row or
// 32-column block of D on the two-kernel path
int64_t grad_chunks(const egm_plan_s* p, int cfg) {
  if (p->epilog != EGM_EPILOG_DRELU_BGRAD) return 0;
  if (p->bias_layout == EGM_BIAS_COL) return cdiv(p->m, p->fused ? kConfigs[cfg].bm : 32);
  return cdiv(p->n, p->fused ? kConfigs[cfg].bn : 32);
}

// tile rows per L2-sharing group actually launched
int32_t effective_group_m(const egm_plan_s* p, int cfg) {
  const int64_t tiles_m = (p->m + kConfigs[cfg].bm - 1) / kConfigs[cfg].bm;
  const int64_t g = p->group_m > 0 ? p->group_m : 4;
  return int32_t(g < tiles_m ? g : (tiles_m > 0 ? tiles_m : 1));
}

void describe(const egm_plan_s* p, char* buf, size_t len) {
  const ConfigInfo& c = kConfigs[p->config];
  static const char* fmt8[2] = {"e4m3", "e5m2"};
  char operands[40];
  if (p->f8 != 0)
    snprintf(operands, sizeof(operands), "%sx%s", fmt8[(p->f8 - 1) & 1], fmt8[(p->f8 - 1) >> 1]);
  else
    snprintf(operands, sizeof(operands), "%s", p->dtype == EGM_F16 ? "fp16" : "bf16");
  snprintf(buf, len,
           "egm m=%lld n=%lld k=%lld operands=%s%s dtype=%s epilog=%s bias=%s path=%s tile=%dx%d kslab=%d waves=%dx%d "
           "mfma=%s lds_ring=%d group_m=%d tiles=%lld workspace=%zu%s",
           (long long)p->m, (long long)p->n, (long long)p->k, operands, p->b_transposed ? " b=[n,k]" : "",
           p->dtype == EGM_F16 ? "fp16" : "bf16",
           epilog_name(p->epilog), p->bias_layout == EGM_BIAS_ROW ? "row(m,1)" : p->bias_layout == EGM_BIAS_COL ? "col(1,n)" : "none",
           p->fused ? "fused" : "unfused(gemm+epilogue)", c.bm, c.bn, p->f8 != 0 ? 2 * c.bk : c.bk, c.wm, c.wn,
           p->f8 != 0 ? "32x32x64" : c.mi == 16 ? "16x16x32" : "32x32x16", c.stages, effective_group_m(p, p->config),
           (long long)(cdiv(p->m, c.bm) * cdiv(p->n, c.bn)), p->workspace_bytes,
           p->autotune_pending ? " autotune=pending" : "");
}

// a strided batch of problems in one launch (grid.y); {1, 0, ...} for one problem
struct Batch {
  int64_t count;
  int64_t stride_a, stride_b, stride_d, stride_aux;
};
constexpr Batch kOne{1, 0, 0, 0, 0};

hipError_t launch_plan(const egm_plan_s* p, int cfg, const void* A, const void* B, void* D, void* aux,
                       void* ws, hipStream_t s, const Batch& bt = kOne) {
  const ConfigInfo& c = kConfigs[cfg];
  const int dt = p->dtype == EGM_F16 ? egm::DT_F16 : egm::DT_BF16;
  const int64_t chunks = grad_chunks(p, cfg);
  float* partial = chunks > 0 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p->product_bytes) : nullptr;
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.bias = p->bias;
  g.R = p->residual;
  g.aux = aux;
  g.partial = partial;
  g.scale_a = p->scale_a;
  g.scale_b = p->scale_b;
  g.stride_a = bt.stride_a;
  g.stride_b = bt.stride_b;
  g.stride_d = bt.stride_d;
  g.stride_aux = bt.stride_aux;
  g.M = int32_t(p->m);
  g.N = int32_t(p->n);
  g.K = int32_t(p->k);
  g.bias_layout = p->bias_layout;
  g.tiles_m = int32_t(cdiv(p->m, c.bm));
  g.tiles_n = int32_t(cdiv(p->n, c.bn));
  g.group_m = effective_group_m(p, cfg);
  const dim3 grid(uint32_t(int64_t(g.tiles_m) * g.tiles_n), uint32_t(bt.count));
  const int epi = epi_of(p->epilog);
  const bool two_kernels = !p->fused && epi != egm::EPI_NONE;
  g.D = two_kernels ? ws : D;
  const int gemm_epi = gemm_epi_of(p);
  const bool b_t = p->b_transposed != 0;
  GemmLaunch gl = p->f8 != 0 ? egm::gemm_launcher_fp8(dt, p->f8, gemm_epi, cfg, b_t)
                             : egm::gemm_launcher(dt, gemm_epi, cfg, b_t);
  if (gl == nullptr) return hipErrorInvalidValue;
  gl(grid, s, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the bias gradient's last step: sum the per-block partials in block order
  auto finish_grad = [&]() {
    int64_t blocks = cdiv(p->grad_len, 64);
    if (blocks > 4096) blocks = 4096;
    egm::launch_bias_grad_finish(dim3(uint32_t(blocks)), s, partial, chunks, p->grad_len,
                                 static_cast<float*>(p->bias_grad));
    return hipGetLastError();
  };
  if (!two_kernels) return epi == egm::EPI_DRELU_BGRAD ? finish_grad() : err;
  EpiArgs e{};
  e.P = ws;
  e.bias = p->bias;
  e.R = p->residual;
  e.D = D;
  e.aux = aux;
  e.M = p->m;
  e.N = int32_t(p->n);
  e.bias_layout = p->bias_layout;
  const int64_t units = p->m * (p->n / 8);
  int64_t blocks = cdiv(units, 256);
  if (blocks > 8 * 1024) blocks = 8 * 1024;
  // the backward two-kernel path applies the mask with the DRELU epilogue
  // kernel, then sums the bias gradient from D
  EpiLaunch el = egm::epi_launcher(dt, epi == egm::EPI_DRELU_BGRAD ? egm::EPI_DRELU : epi);
  if (el == nullptr) return hipErrorInvalidValue;
  el(dim3(uint32_t(blocks)), s, e);
  err = hipGetLastError();
  if (err != hipSuccess || epi != egm::EPI_DRELU_BGRAD) return err;
  const int64_t punits = p->bias_layout == EGM_BIAS_COL ? cdiv(p->m, 32) * (p->n / 8) : p->m * cdiv(p->n, 32);
  int64_t pblocks = cdiv(punits, 256);
  if (pblocks > 8 * 1024) pblocks = 8 * 1024;
  egm::partials_launcher(dt)(dim3(uint32_t(pblocks)), s, D, p->m, int32_t(p->n), p->bias_layout, partial);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return finish_grad();
}

// Time every config once (after one warm-up launch each) on the caller's
// stream and keep the fastest.  Runs on the first execute of an autotune plan.
hipError_t autotune(egm_plan_s* p, const void* A, const void* B, void* D, void* aux, void* ws, hipStream_t s) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  err = hipEventCreate(&e1);
  if (err != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  float best = -1.0f;
  int best_cfg = p->config;
  for (int c = 0; c < kNumConfigs && err == hipSuccess; ++c) {
    if (!grid_fits(p->m, p->n, c) || !config_built(c, p->f8 != 0)) continue;
    err = launch_plan(p, c, A, B, D, aux, ws, s);
    if (err != hipSuccess) break;
    err = hipEventRecord(e0, s);
    for (int r = 0; r < 3 && err == hipSuccess; ++r) err = launch_plan(p, c, A, B, D, aux, ws, s);
    if (err == hipSuccess) err = hipEventRecord(e1, s);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess && (best < 0.0f || ms < best)) {
      best = ms;
      best_cfg = c;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err == hipSuccess) {
    p->config.store(best_cfg, std::memory_order_relaxed);
    p->autotune_pending.store(0, std::memory_order_release);
  }
  return err;
}

// The first execute of an autotune plan times every config and waits for the
// events on the host, so it cannot be recorded into a graph: on a capturing
// stream it is refused (EGM_ERR_NOT_SUPPORTED) and the plan stays pending.
// Executes from several threads run the tuning once.
egm_status_t tune_if_pending(egm_plan_s* p, const void* A, const void* B, void* D, void* aux, void* ws,
                             hipStream_t s) {
  if (!p->autotune_pending.load(std::memory_order_acquire)) return EGM_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return EGM_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return EGM_ERR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(p->tune_mu);
  if (!p->autotune_pending.load(std::memory_order_acquire)) return EGM_OK;
  return autotune(p, A, B, D, aux, ws, s) == hipSuccess ? EGM_OK : EGM_ERR_HIP;
}

// Validation and construction shared by egm_plan (f8 = 0) and egm_plan_fp8.
egm_status_t plan_impl(egm_plan_t* out, int64_t m, int64_t n, int64_t k, egm_dtype_t dtype, int32_t f8,
                       const float* scale_a, const float* scale_b, egm_epilog_t epilog,
                       const egm_epilog_inputs_t* in, const egm_plan_options_t* opt) {
  if (out == nullptr) return EGM_ERR_INVALID_VALUE;
  *out = nullptr;
  if (m < 0 || n < 0 || k < 0) return EGM_ERR_SHAPE;
  const int64_t row_elems = f8 != 0 ? 16 : 8;  // elements per 16-byte operand row piece
  if ((n % row_elems) != 0 || (k % row_elems) != 0) return EGM_ERR_SHAPE;
  if (n > kMaxNK || k > kMaxNK || m > int64_t(0x7fffffff)) return EGM_ERR_SHAPE;
  if (dtype != EGM_F16 && dtype != EGM_BF16) return EGM_ERR_DTYPE;
  if (int(epilog) < 0 || int(epilog) >= kNumEpi) return EGM_ERR_INVALID_VALUE;
  if (f8 != 0 && (epilog == EGM_EPILOG_DRELU || epilog == EGM_EPILOG_DRELU_BGRAD)) return EGM_ERR_NOT_SUPPORTED;
  if ((reinterpret_cast<uintptr_t>(scale_a) & 3u) != 0 || (reinterpret_cast<uintptr_t>(scale_b) & 3u) != 0)
    return EGM_ERR_ALIGNMENT;

  const void* bias = nullptr;
  const void* residual = nullptr;
  void* bias_grad = nullptr;
  int32_t layout = EGM_BIAS_NONE;
  if (in != nullptr && in->bias_grad != nullptr && epilog != EGM_EPILOG_DRELU_BGRAD)
    return EGM_ERR_INVALID_VALUE;  // a bias gradient only belongs to DRELU_BGRAD
  if (epilog == EGM_EPILOG_DEFAULT || epilog == EGM_EPILOG_DRELU) {
    if (in != nullptr && (in->bias != nullptr || in->residual != nullptr || in->bias_layout != EGM_BIAS_NONE))
      return EGM_ERR_INVALID_VALUE;  // DEFAULT and DRELU take no epilog inputs
  } else if (epilog == EGM_EPILOG_DRELU_BGRAD) {
    if (in == nullptr || in->bias_grad == nullptr) return EGM_ERR_INVALID_VALUE;
    if (in->bias != nullptr || in->residual != nullptr) return EGM_ERR_INVALID_VALUE;
    if (in->bias_layout != EGM_BIAS_ROW && in->bias_layout != EGM_BIAS_COL) return EGM_ERR_SHAPE;
    if (!aligned16(in->bias_grad)) return EGM_ERR_ALIGNMENT;
    bias_grad = in->bias_grad;
    layout = in->bias_layout;
  } else {
    if (in == nullptr || in->bias == nullptr) return EGM_ERR_INVALID_VALUE;
    if (in->bias_layout != EGM_BIAS_ROW && in->bias_layout != EGM_BIAS_COL) return EGM_ERR_SHAPE;
    if (!aligned16(in->bias)) return EGM_ERR_ALIGNMENT;
    bias = in->bias;
    layout = in->bias_layout;
    if (epilog == EGM_EPILOG_BIAS_RESIDUAL) {
      if (in->residual == nullptr) return EGM_ERR_INVALID_VALUE;
      if (!aligned16(in->residual)) return EGM_ERR_ALIGNMENT;
      residual = in->residual;
    } else if (in->residual != nullptr) {
      return EGM_ERR_INVALID_VALUE;  // a residual only belongs to BIAS_RESIDUAL
    }
  }

  int32_t fused = 1, force = -1, tune = 0, group_m = 0, b_transposed = 0;
  if (opt != nullptr) {
    if (opt->b_transposed != 0 && opt->b_transposed != 1) return EGM_ERR_INVALID_VALUE;
    b_transposed = opt->b_transposed;
    if (opt->fused != 0 && opt->fused != 1) return EGM_ERR_INVALID_VALUE;
    if (opt->force_config < -1 || opt->force_config >= kNumConfigs) return EGM_ERR_INVALID_VALUE;
    if (opt->autotune != 0 && opt->autotune != 1) return EGM_ERR_INVALID_VALUE;
    if (opt->group_m < 0 || opt->group_m > 4096) return EGM_ERR_INVALID_VALUE;
    if (opt->autotune && opt->force_config >= 0) return EGM_ERR_INVALID_VALUE;
    fused = opt->fused;
    force = opt->force_config;
    tune = opt->autotune;
    group_m = opt->group_m;
  }

  std::shared_ptr<egm_plan_s> owner;
  try {
    owner = std::make_shared<egm_plan_s>();
  } catch (const std::bad_alloc&) {
    return EGM_ERR_NO_MEMORY;
  }
  egm_plan_s* p = owner.get();
  p->m = m;
  p->n = n;
  p->k = k;
  p->dtype = dtype;
  p->epilog = epilog;
  p->bias = bias;
  p->bias_layout = layout;
  p->residual = residual;
  p->bias_grad = bias_grad;
  p->f8 = f8;
  p->scale_a = scale_a;
  p->scale_b = scale_b;
  p->b_transposed = b_transposed;
  p->fused = fused;
  p->config = force >= 0 ? force : choose_config(m, n, k, f8 != 0, gemm_epi_of(p), b_transposed != 0);
  p->chosen_per_shape = force < 0 && !tune;
  // the launch must fit one grid dimension and the config exist for the
  // operand type (autotuning tries only such configs, and the per-shape
  // choice always is one)
  if (p->config < 0 || !grid_fits(m, n, p->config) || !config_built(p->config, f8 != 0))
    return EGM_ERR_NOT_SUPPORTED;
  p->group_m = group_m;
  p->autotune_pending = tune;
  // workspace: the two-kernel path's product P, then (DRELU_BGRAD) the fp32
  // partial sums, sized for every config the plan may launch (all of them
  // while autotuning is pending)
  p->product_bytes = (!fused && epilog != EGM_EPILOG_DEFAULT) ? (size_t(m) * size_t(n) * 2u + 255u) & ~size_t(255) : 0u;
  p->grad_len = epilog == EGM_EPILOG_DRELU_BGRAD ? (layout == EGM_BIAS_COL ? n : m) : 0;
  int64_t max_chunks = 0;
  for (int c = 0; c < kNumConfigs; ++c) {
    if ((tune && grid_fits(m, n, c) && config_built(c, f8 != 0)) || c == p->config) {
      const int64_t ch = grad_chunks(p, c);
      if (ch > max_chunks) max_chunks = ch;
    }
  }
  p->workspace_bytes = p->product_bytes + size_t(max_chunks) * size_t(p->grad_len) * 4u;
  if (const char* log = std::getenv("EGM_LOG"); log != nullptr && log[0] == '1') {
    char buf[512];
    describe(p, buf, sizeof(buf));
    std::fprintf(stderr, "[egm] plan: %s\n", buf);
  }
  try {
    *out = register_plan(std::move(owner));
  } catch (const std::bad_alloc&) {
    return EGM_ERR_NO_MEMORY;
  }
  return EGM_OK;
}

// Scratch of egm_execute_no_alloc: the workspace (the two-kernel path's
// product, the bias gradient's per-tile partial sums) for callers that cannot
// allocate device memory.  Each GPU that runs the library holds its own copy
// until the process ends.  Host code never passes this name to a kernel or a
// copy (on the host it is only a stand-in for the symbol): it uses the
// device address that scratch_address() obtains once per device.
static __device__ __align__(256) uint8_t scratch[EGM_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the calling thread's current device, looked
// up on the first call from that device (with it current) and kept.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

// egm_execute (own_scratch = false: the caller's workspace) and
// egm_execute_no_alloc (own_scratch = true: the library's static scratch on
// the current device, which the stream must belong to).
egm_status_t execute_impl(egm_plan_s* p, const void* A, const void* B, void* D, void* aux, void* workspace,
                          size_t workspace_bytes, void* stream, bool own_scratch) {
  // (own_scratch: the workspace arguments are unused)
  const bool need_aux = p->epilog == EGM_EPILOG_RELU_AUX_BIAS || p->epilog == EGM_EPILOG_DRELU ||
                        p->epilog == EGM_EPILOG_DRELU_BGRAD;
  const bool empty = p->m == 0 || p->n == 0;
  // an empty problem has an empty mask, which may come as NULL
  if (need_aux ? (aux == nullptr && !empty) : aux != nullptr) return EGM_ERR_INVALID_VALUE;
  if (own_scratch) {
    if (p->workspace_bytes > size_t(EGM_NO_ALLOC_SCRATCH_BYTES)) return EGM_ERR_SCRATCH_LIMIT;
    // tuning creates and waits on events
    if (p->autotune_pending.load(std::memory_order_acquire)) return EGM_ERR_NOT_SUPPORTED;
  } else if (p->workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < p->workspace_bytes)) {
    return EGM_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (empty) {
    // empty output: nothing to compute, but a bias gradient of a non-empty
    // axis is a sum of nothing: zeros
    // (written by the finish kernel over zero chunks, not a memset, so the
    // call stays capturable in a graph)
    if (p->bias_grad != nullptr && p->grad_len > 0) {
      if (!aligned16(p->bias_grad)) return EGM_ERR_ALIGNMENT;
      int64_t blocks = cdiv(p->grad_len, 64);
      if (blocks > 4096) blocks = 4096;
      egm::launch_bias_grad_finish(dim3(uint32_t(blocks)), s, nullptr, 0, p->grad_len,
                                   static_cast<float*>(p->bias_grad));
      return hipGetLastError() == hipSuccess ? EGM_OK : EGM_ERR_HIP;
    }
    return EGM_OK;
  }
  if (D == nullptr) return EGM_ERR_INVALID_VALUE;
  if (p->k > 0 && (A == nullptr || B == nullptr)) return EGM_ERR_INVALID_VALUE;
  if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(D) || (aux && !aligned16(aux)) ||
      (!own_scratch && p->workspace_bytes > 0 && !aligned16(workspace)))
    return EGM_ERR_ALIGNMENT;
  if (std::getenv("EGM_FAIL_INJECT") != nullptr && std::strcmp(std::getenv("EGM_FAIL_INJECT"), "launch") == 0)
    return EGM_ERR_HIP;  // host-forced launch-error path, for tests of the error handling
  if (own_scratch && p->workspace_bytes > 0) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess) return EGM_ERR_HIP;
    if (sdev != cur) return EGM_ERR_INVALID_VALUE;  // the scratch used is the current device's
    if (scratch_address(&workspace) != hipSuccess) return EGM_ERR_HIP;
  }
  const egm_status_t tuned = tune_if_pending(p, A, B, D, aux, workspace, s);
  if (tuned != EGM_OK) return tuned;
  const hipError_t err = launch_plan(p, p->config, A, B, D, aux, workspace, s);
  return err == hipSuccess ? EGM_OK : EGM_ERR_HIP;
}

}  // namespace

extern "C" {

egm_status_t egm_plan(egm_plan_t* out, int64_t m, int64_t n, int64_t k, egm_dtype_t dtype,
                      egm_epilog_t epilog, const egm_epilog_inputs_t* in, const egm_plan_options_t* opt) {
  return plan_impl(out, m, n, k, dtype, 0, nullptr, nullptr, epilog, in, opt);
}

egm_status_t egm_plan_fp8(egm_plan_t* out, int64_t m, int64_t n, int64_t k, egm_fp8_format_t a_format,
                          egm_fp8_format_t b_format, egm_dtype_t out_dtype, const float* scale_a,
                          const float* scale_b, egm_epilog_t epilog, const egm_epilog_inputs_t* in,
                          const egm_plan_options_t* opt) {
  if (out == nullptr) return EGM_ERR_INVALID_VALUE;
  *out = nullptr;
  const bool known = (a_format == EGM_E4M3 || a_format == EGM_E5M2) && (b_format == EGM_E4M3 || b_format == EGM_E5M2);
  if (!known) return EGM_ERR_DTYPE;
  const int32_t f8 = 1 + int32_t(a_format) + 2 * int32_t(b_format);
  return plan_impl(out, m, n, k, out_dtype, f8, scale_a, scale_b, epilog, in, opt);
}

egm_status_t egm_execute(egm_plan_t plan, const void* A, const void* B, void* D, void* aux, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const std::shared_ptr<egm_plan_s> ref = lookup(plan);
  if (ref == nullptr) return EGM_ERR_INVALID_PLAN;
  return execute_impl(ref.get(), A, B, D, aux, workspace, workspace_bytes, stream, false);
}

egm_status_t egm_execute_no_alloc(egm_plan_t plan, const void* A, const void* B, void* D, void* aux,
                                  void* stream) {
  const std::shared_ptr<egm_plan_s> ref = lookup(plan);
  if (ref == nullptr) return EGM_ERR_INVALID_PLAN;
  return execute_impl(ref.get(), A, B, D, aux, nullptr, 0, stream, true);
}

egm_status_t egm_execute_strided(egm_plan_t plan, int64_t batch, const void* A, int64_t stride_a, const void* B,
                                 int64_t stride_b, void* D, int64_t stride_d, void* aux, int64_t stride_aux,
                                 void* stream) {
  const std::shared_ptr<egm_plan_s> ref = lookup(plan);
  if (ref == nullptr) return EGM_ERR_INVALID_PLAN;
  egm_plan_s* p = ref.get();
  if (batch < 0 || batch > 65535) return EGM_ERR_INVALID_VALUE;
  if (!p->fused || p->epilog == EGM_EPILOG_DRELU_BGRAD) return EGM_ERR_NOT_SUPPORTED;
  const bool need_aux = p->epilog == EGM_EPILOG_RELU_AUX_BIAS || p->epilog == EGM_EPILOG_DRELU;
  const bool empty = batch == 0 || p->m == 0 || p->n == 0;
  if (need_aux ? (aux == nullptr && !empty) : aux != nullptr) return EGM_ERR_INVALID_VALUE;
  if (stride_a < 0 || stride_b < 0 || stride_d < 0 || stride_aux < 0) return EGM_ERR_INVALID_VALUE;
  // the outputs of different problems must not overlap
  if (batch > 1 && (stride_d < p->m * p->n || (need_aux && stride_aux < p->m * (p->n / 8))))
    return EGM_ERR_INVALID_VALUE;
  if (empty) return EGM_OK;
  if (D == nullptr) return EGM_ERR_INVALID_VALUE;
  if (p->k > 0 && (A == nullptr || B == nullptr)) return EGM_ERR_INVALID_VALUE;
  // every problem's operands keep the 16-byte alignment of the first
  const int64_t es = p->f8 != 0 ? 1 : 2;
  if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(D) || (aux && !aligned16(aux)) ||
      (stride_a * es) % 16 != 0 || (stride_b * es) % 16 != 0 || (stride_d * 2) % 16 != 0 || stride_aux % 16 != 0)
    return EGM_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // tuned on the first problem
  const egm_status_t tuned = tune_if_pending(p, A, B, D, aux, nullptr, s);
  if (tuned != EGM_OK) return tuned;
  // a per-shape choice is made again for the whole batch (the tiles of all
  // its problems share the CUs); a forced or autotuned config is kept
  int cfg = p->config;
  if (p->chosen_per_shape && batch > 1) {
    const int c = choose_config(p->m, p->n, p->k, p->f8 != 0, gemm_epi_of(p), p->b_transposed != 0, batch);
    if (c >= 0) cfg = c;
  }
  const hipError_t err =
      launch_plan(p, cfg, A, B, D, aux, nullptr, s, Batch{batch, stride_a, stride_b, stride_d, stride_aux});
  return err == hipSuccess ? EGM_OK : EGM_ERR_HIP;
}

egm_status_t egm_free(egm_plan_t plan) {
  if (plan == nullptr) return EGM_OK;
  return unregister(plan) ? EGM_OK : EGM_ERR_INVALID_PLAN;
}

size_t egm_plan_workspace_bytes(egm_plan_t plan) {
  const std::shared_ptr<egm_plan_s> p = lookup(plan);
  return p != nullptr ? p->workspace_bytes : 0;
}

egm_status_t egm_plan_describe(egm_plan_t plan, char* buf, size_t len) {
  const std::shared_ptr<egm_plan_s> p = lookup(plan);
  if (p == nullptr) return EGM_ERR_INVALID_PLAN;
  if (buf == nullptr || len == 0) return EGM_ERR_INVALID_VALUE;
  describe(p.get(), buf, len);
  return EGM_OK;
}

int32_t egm_plan_config(egm_plan_t plan) {
  const std::shared_ptr<egm_plan_s> p = lookup(plan);
  return p != nullptr ? p->config.load(std::memory_order_relaxed) : -1;
}

int32_t egm_num_configs(void) { return kNumConfigs; }

egm_status_t egm_config_describe(int32_t config, char* buf, size_t len) {
  if (config < 0 || config >= kNumConfigs) return EGM_ERR_INVALID_VALUE;
  if (buf == nullptr || len == 0) return EGM_ERR_INVALID_VALUE;
  const ConfigInfo& c = kConfigs[config];
  snprintf(buf, len, "tile=%dx%d kslab=%d waves=%dx%d wave_tile=%dx%d mfma=%s lds_ring=%d lds_bytes=%d%s", c.bm,
           c.bn, c.bk, c.wm, c.wn, c.bm / c.wm, c.bn / c.wn, c.mi == 16 ? "16x16x32" : "32x32x16", c.stages,
           c.stages * (c.bm + c.bn) * c.bk * 2, c.mi == 16 ? " operands=16-bit" : "");
  return EGM_OK;
}

const char* egm_status_string(egm_status_t s) {
  switch (s) {
    case EGM_OK: return "EGM_OK";
    case EGM_ERR_INVALID_VALUE: return "EGM_ERR_INVALID_VALUE: invalid argument";
    case EGM_ERR_NOT_SUPPORTED: return "EGM_ERR_NOT_SUPPORTED: not supported";
    case EGM_ERR_SHAPE: return "EGM_ERR_SHAPE: invalid shape (dims >= 0, n and k multiples of 8 (16 for fp8), n,k <= 2^21)";
    case EGM_ERR_DTYPE: return "EGM_ERR_DTYPE: dtype must be fp16 or bf16";
    case EGM_ERR_ALIGNMENT: return "EGM_ERR_ALIGNMENT: device pointers must be 16-byte aligned";
    case EGM_ERR_INVALID_PLAN: return "EGM_ERR_INVALID_PLAN: NULL, freed or foreign plan handle";
    case EGM_ERR_HIP: return "EGM_ERR_HIP: HIP runtime error at launch";
    case EGM_ERR_NO_MEMORY: return "EGM_ERR_NO_MEMORY: host allocation failed";
    case EGM_ERR_WORKSPACE: return "EGM_ERR_WORKSPACE: workspace missing or too small";
    case EGM_ERR_SCRATCH_LIMIT:
      return "EGM_ERR_SCRATCH_LIMIT: the plan needs more workspace than the static scratch of "
             "egm_execute_no_alloc holds (EGM_NO_ALLOC_SCRATCH_BYTES)";
  }
  return "EGM: unknown status";
}

egm_status_t egm_layernorm(int64_t rows, int64_t cols, egm_dtype_t dtype, const void* x, const void* residual,
                           const void* gamma, const void* beta, float eps, void* y, float* mean, float* rstd,
                           void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return EGM_ERR_SHAPE;
  constexpr int64_t kMaxCols = int64_t(egm::kLnConfigs[egm::kNumLnConfigs - 1].tpr) *
                               egm::kLnConfigs[egm::kNumLnConfigs - 1].cpt * 8;
  if (cols > kMaxCols) return EGM_ERR_SHAPE;
  if (dtype != EGM_F16 && dtype != EGM_BF16) return EGM_ERR_DTYPE;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return EGM_ERR_INVALID_VALUE;  // also rejects NaN
  if (rows == 0) return EGM_OK;
  if (x == nullptr || y == nullptr) return EGM_ERR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(y) || (residual && !aligned16(residual)) || (gamma && !aligned16(gamma)) ||
      (beta && !aligned16(beta)) || (reinterpret_cast<uintptr_t>(mean) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(rstd) & 3u) != 0)
    return EGM_ERR_ALIGNMENT;
  int cfg = 0;
  while (int64_t(egm::kLnConfigs[cfg].tpr) * egm::kLnConfigs[cfg].cpt * 8 < cols) ++cfg;
  // one grid dimension of 256-thread workgroups: at most 2^32 - 1 work-items
  const int64_t rows_per_wg = 256 / egm::kLnConfigs[cfg].tpr;
  const int64_t wgs = cdiv(rows, rows_per_wg);
  if (wgs * 256 > int64_t(0xffffffff)) return EGM_ERR_NOT_SUPPORTED;
  const egm::LnLaunch launch = dtype == EGM_F16 ? egm::layernorm_launcher_f16(cfg, residual != nullptr)
                                                : egm::layernorm_launcher_bf16(cfg, residual != nullptr);
  if (launch == nullptr) return EGM_ERR_NOT_SUPPORTED;
  egm::LnArgs a{};
  a.x = x;
  a.r = residual;
  a.gamma = gamma;
  a.beta = beta;
  a.y = y;
  a.mean = mean;
  a.rstd = rstd;
  a.M = rows;
  a.N = int32_t(cols);
  a.eps = eps;
  launch(dim3(uint32_t(wgs)), reinterpret_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? EGM_OK : EGM_ERR_HIP;
}

int32_t egm_abi_version(void) { return EGM_ABI_VERSION; }

}  // extern "C"
