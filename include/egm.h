/*
 * egm.h - fused dense GEMM + epilogue for AMD Instinct MI355X (gfx950).
 *
 *   D = epilogue(A . B),  A [m,k], B [k,n], D [m,n], all row-major, one 16-bit
 *   dtype (fp16 or bf16) for A, B, bias, residual and D (egm_plan_fp8: fp8
 *   A and B with per-tensor scales, 16-bit bias, residual and D); products
 *   accumulate in fp32 and the epilogue runs on the fp32 accumulators before
 *   the single round-to-nearest-even conversion to the output dtype.
 *
 * Pages this interface follows (cited by title):
 *   [bias-fusion] "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
 *                 (blog.hotdry.top, 2025-09-22): the stateful Matmul object
 *                 (construct, plan with an epilog and a dict of epilog inputs,
 *                 execute, free) in the body's code example; the epilog names
 *                 BIAS / RELU_BIAS / RELU_AUX_BIAS; the checklist after the
 *                 example (matching dtypes, bias shaped (m,1) or (1,n), free
 *                 releases the plan, autotuning through options).
 *   [bindings]    "nvmath-python：cuBLAS与cuSOLVER的Python绑定加速ML线性代数"
 *                 (blog.hotdry.top, 2025-09-19), body, checklist items 2-3:
 *                 plan() chooses the algorithm, execute() is non-blocking and
 *                 the caller synchronises the stream, the algorithm choice can
 *                 be inspected.
 *   [op-fusion]   "模型推理中的算子融合优化从LayerNorm到残差连接的图级优化"
 *                 (wmrh.cn news 429806) §一 (FFN chain matmul -> bias -> GELU)
 *                 and §三 (residual added while the producer's output is still
 *                 in registers).
 *
 * Ownership: the caller owns every device buffer (A, B, D, bias, residual,
 * aux mask, workspace).  The library never allocates device memory.  A plan is
 * a small host object owned by the library from egm_plan until egm_free.
 * Epilog inputs (bias, residual) are bound at plan time, as the pages bind them
 * in plan(); they must stay valid for every execute of that plan.  A, B, D and
 * the mask are bound per execute, so one plan serves many batches.
 *
 * Errors: every function returns a status; nothing is thrown across the ABI.
 * All argument checks run on the host before any HIP call.  There is no
 * implicit dtype conversion.  egm_execute is asynchronous and stream-ordered:
 * it returns EGM_ERR_HIP only when the launch itself fails; a device fault
 * shows at the caller's next synchronisation of the stream.  Plans are
 * immutable after egm_plan (but for the one-time choice of a pending
 * autotune), so executes of one plan on several streams may overlap (their
 * outputs must not).
 */
#ifndef EGM_H_
#define EGM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EGM_ABI_VERSION 7

/* Every enum of this interface is int32_t-sized.  A C caller may pass any
 * int32_t where one is expected (unknown values are rejected with a status);
 * the C++ side fixes the underlying type so that such values are well-defined
 * there too. */
#ifdef __cplusplus
#define EGM_ENUM(name) enum name : int32_t
#else
#define EGM_ENUM(name) enum name
#endif

typedef EGM_ENUM(egm_status_t) {
  EGM_OK = 0,
  EGM_ERR_INVALID_VALUE = 1, /* NULL pointer, unknown enum, bad option */
  EGM_ERR_NOT_SUPPORTED = 2, /* valid request outside what v1 implements */
  EGM_ERR_SHAPE = 3,         /* negative dims, n or k not a multiple of 8 (16 for fp8), too large */
  EGM_ERR_DTYPE = 4,         /* dtype other than fp16 / bf16, or an unknown fp8 format */
  EGM_ERR_ALIGNMENT = 5,     /* device pointer not 16-byte aligned (fp8 scales: 4-byte) */
  EGM_ERR_INVALID_PLAN = 6,  /* NULL, freed or foreign plan handle */
  EGM_ERR_HIP = 7,           /* the HIP runtime reported an error at launch */
  EGM_ERR_NO_MEMORY = 8,     /* host allocation of the plan failed */
  EGM_ERR_WORKSPACE = 9,     /* workspace missing or smaller than egm_plan_workspace_bytes */
  EGM_ERR_SCRATCH_LIMIT = 10 /* egm_execute_no_alloc: the plan needs more workspace than
                                EGM_NO_ALLOC_SCRATCH_BYTES */
} egm_status_t;

/* Bytes of the static scratch behind egm_execute_no_alloc (per GPU). */
#define EGM_NO_ALLOC_SCRATCH_BYTES (32u << 20)

typedef EGM_ENUM(egm_dtype_t) {
  EGM_F16 = 0,  /* IEEE binary16 */
  EGM_BF16 = 1  /* bfloat16 (upper half of binary32) */
} egm_dtype_t;

/* fp8 operand formats of egm_plan_fp8 (the OCP 8-bit floats gfx950 implements). */
typedef EGM_ENUM(egm_fp8_format_t) {
  EGM_E4M3 = 0, /* 4 exponent bits (bias 7), 3 mantissa bits; no infinities; largest 448 */
  EGM_E5M2 = 1  /* 5 exponent bits (bias 15), 2 mantissa bits; IEEE inf / NaN; largest 57344 */
} egm_fp8_format_t;

/*
 * Epilogues.  Z = A.B + bias (fp32, bias broadcast per egm_bias_layout_t).
 *   DEFAULT        D = A.B                    (no epilog inputs)
 *   BIAS           D = Z                      [bias-fusion] body, code example
 *   RELU_BIAS      D = max(Z, 0)              [bias-fusion] body, before the example
 *   GELU_BIAS      D = 0.5 Z (1 + tanh(sqrt(2/pi) (Z + 0.044715 Z^3)))
 *                                             ([op-fusion] §一 FFN chain; the
 *                                             tanh form of Hendrycks & Gimpel)
 *   RELU_AUX_BIAS  D = max(Z, 0) and aux[i, j/8] bit (j%8) = (Z[i,j] > 0)
 *                                             [bias-fusion] body, limitations
 *                                             paragraph (mask for backward)
 *   BIAS_RESIDUAL  D = Z + R, R [m,n] row-major   [op-fusion] §三
 *
 * Backward epilogues (consumers of the RELU_AUX_BIAS mask; [bias-fusion] body:
 * the training paragraph (the forward must leave the mask backward needs) and
 * the closing paragraph (dBias as an epilogue to come)).  Here A.B is the
 * gradient reaching the ReLU output, dZ its part that passes the ReLU:
 *   DRELU          D = dZ = (A.B) where the mask bit is 1, else 0
 *                  (aux at execute is the INPUT mask, as RELU_AUX_BIAS wrote it)
 *   DRELU_BGRAD    D as DRELU, and the bias gradient of the forward bias:
 *                  bias_layout COL ((1,n) bias): grad[j] = sum_i dZ[i,j], n values;
 *                  bias_layout ROW ((m,1) bias): grad[i] = sum_j dZ[i,j], m values;
 *                  summed in fp32 from the unrounded dZ, written as fp32 to
 *                  egm_epilog_inputs_t.bias_grad
 * No bias is added in either backward epilogue.
 */
typedef EGM_ENUM(egm_epilog_t) {
  EGM_EPILOG_DEFAULT = 0,
  EGM_EPILOG_BIAS = 1,
  EGM_EPILOG_RELU_BIAS = 2,
  EGM_EPILOG_GELU_BIAS = 3,
  EGM_EPILOG_RELU_AUX_BIAS = 4,
  EGM_EPILOG_BIAS_RESIDUAL = 5,
  EGM_EPILOG_DRELU = 6,
  EGM_EPILOG_DRELU_BGRAD = 7
} egm_epilog_t;

/* Bias shapes accepted by the pages ([bias-fusion] body, shape item of the
 * checklist): (m,1) adds bias[i] to row i, (1,n) adds bias[j] to column j. */
typedef EGM_ENUM(egm_bias_layout_t) {
  EGM_BIAS_NONE = 0,
  EGM_BIAS_ROW = 1, /* shape (m,1): m elements */
  EGM_BIAS_COL = 2  /* shape (1,n): n elements */
} egm_bias_layout_t;

/* Named epilog operands (the pages' epilog_inputs dict).  Device pointers,
 * caller-owned, 16-byte aligned, in the plan's dtype unless stated. */
typedef struct egm_epilog_inputs_t {
  const void* bias;      /* required for BIAS .. BIAS_RESIDUAL; NULL for DEFAULT and
                            the backward epilogues */
  int32_t bias_layout;   /* egm_bias_layout_t; for DRELU_BGRAD it selects the
                            gradient's axis (ROW: m values, COL: n values) */
  const void* residual;  /* [m,n] row-major; required iff BIAS_RESIDUAL, else NULL */
  void* bias_grad;       /* OUTPUT, fp32 (not the plan's dtype), m or n values;
                            required iff DRELU_BGRAD, else NULL */
} egm_epilog_inputs_t;

/* Plan options ([bias-fusion] checklist: autotuning through options). */
typedef struct egm_plan_options_t {
  int32_t fused;         /* 1 (default): one kernel.  0: the two-kernel path kept
                            for measurement (GEMM writes P = round(A.B) to the
                            workspace, a second kernel applies the epilogue). */
  int32_t force_config;  /* -1 (default): per-shape choice; else a tile-config id
                            0 .. egm_num_configs()-1 */
  int32_t autotune;      /* 0 (default); 1: the first execute times every tile
                            config that fits on the caller's stream and
                            buffers (each launched 4 times), keeps the fastest,
                            then launches it: that execute waits on the host
                            for the timings, and on a stream that is being
                            captured into a graph it returns
                            EGM_ERR_NOT_SUPPORTED with the plan still pending
                            (run it once before capture).  Concurrent first
                            executes tune once. */
  int32_t group_m;       /* 0 (default): per-shape choice; else tile rows per
                            L2-sharing group in the workgroup order */
  int32_t b_transposed;  /* 0 (default): B is [k,n] row-major.  1: B is given
                            transposed, as [n,k] row-major (B^T; the layout of
                            a linear layer's [out, in] weight), which the
                            kernel streams like A.  Strided batches advance B
                            by stride_b elements either way. */
} egm_plan_options_t;

typedef struct egm_plan_s* egm_plan_t;

/*
 * egm_plan - validate a problem and choose a kernel configuration.
 *   out     receives the plan handle (set to NULL on error).
 *   m, n, k problem size; m >= 0, n >= 0, k >= 0; n and k multiples of 8
 *           (16-byte rows); n, k <= 2^21; m <= 2^31-1.  m == 0 or n == 0 is an
 *           empty problem (execute does nothing); k == 0 gives D = epilogue(bias).
 *   dtype   EGM_F16 or EGM_BF16, shared by every operand and the output.
 *   epilog  egm_epilog_t.
 *   in      epilog inputs (may be NULL for DEFAULT and DRELU).  RELU_AUX_BIAS
 *           and the backward epilogues need n % 8 == 0 (already required) for
 *           whole mask bytes.
 *   opt     NULL for defaults.
 * A launch is one workgroup per output tile in one grid dimension, which holds
 * at most 2^32 - 1 work-items: the per-shape choice and autotuning consider
 * only the configs whose grid fits (for very tall, narrow problems that
 * excludes the small tiles), and a forced config whose grid does not fit, or
 * a shape no config fits, gives EGM_ERR_NOT_SUPPORTED.
 * No device work and no HIP call.
 */
egm_status_t egm_plan(egm_plan_t* out, int64_t m, int64_t n, int64_t k, egm_dtype_t dtype,
                      egm_epilog_t epilog, const egm_epilog_inputs_t* in,
                      const egm_plan_options_t* opt);

/*
 * egm_plan_fp8 - as egm_plan, with fp8 operands and per-tensor scales
 * ([bias-fusion] body: the data-type item of the checklist lists FP8 among the
 * supported types; the closing paragraph names FP8 among the features to come).
 *   D = epilogue(scale_a * scale_b * (A8 . B8) + bias)
 *   a_format, b_format  egm_fp8_format_t of A [m,k] and B [k,n] (one byte per
 *           element, row-major); any pairing.
 *   out_dtype  EGM_F16 or EGM_BF16: the type of the bias, the residual and D
 *           (the page's same-type rule is read as covering the two operands).
 *   scale_a, scale_b  device pointers to one fp32 each (4-byte aligned), the
 *           dequantisation scales (A = scale_a * A8); read by every execute at
 *           its start, in stream order, so a kernel earlier on the stream may
 *           write them; NULL means 1.  They must stay valid for every execute.
 *   m, n, k as egm_plan, but n and k multiples of 16 (16-byte operand rows).
 *   epilog  DEFAULT .. BIAS_RESIDUAL; the backward epilogues return
 *           EGM_ERR_NOT_SUPPORTED.
 * Products of two fp8 values are exact in fp32 and accumulate in fp32; the
 * scale is one fp32 multiply of the accumulator before the bias.  execute,
 * free, describe and the workspace query work as for egm_plan's plans.
 * No device work and no HIP call.
 */
egm_status_t egm_plan_fp8(egm_plan_t* out, int64_t m, int64_t n, int64_t k, egm_fp8_format_t a_format,
                          egm_fp8_format_t b_format, egm_dtype_t out_dtype, const float* scale_a,
                          const float* scale_b, egm_epilog_t epilog, const egm_epilog_inputs_t* in,
                          const egm_plan_options_t* opt);

/*
 * egm_execute - enqueue the plan on a HIP stream (asynchronous)
 * ([bias-fusion] body, code example: execute() after plan(); [bindings] body,
 * checklist item 2: execute is non-blocking and ordered on the caller's
 * stream, which the caller synchronises).
 *   A     [m,k] device, row-major.          B [k,n] device, row-major ([n,k] row-major
 *         with the b_transposed option).
 *   D     [m,n] device, row-major output.
 *   aux   [m, n/8] uint8 device mask: the OUTPUT of RELU_AUX_BIAS and the INPUT
 *         of DRELU / DRELU_BGRAD; required for those three, else NULL.
 *         Bit (j%8) of byte aux[i*(n/8) + j/8] is 1 iff Z[i,j] > 0 (strict;
 *         least-significant bit = lowest column).
 *   workspace, workspace_bytes: scratch of at least egm_plan_workspace_bytes()
 *         (0 for a fused forward plan; per-tile fp32 partial sums for
 *         DRELU_BGRAD; plus m*n*2 bytes for the product on the two-kernel
 *         path); may be NULL when that is 0.  Its contents need no
 *         initialisation and are garbage afterwards.
 *   stream  a hipStream_t (NULL = the null stream).
 * All pointers 16-byte aligned.  A, B, bias, residual must not alias D or aux;
 * the bias gradient must not alias anything else.  DRELU_BGRAD is two
 * launches on the stream (the GEMM with its per-tile sums, then their
 * reduction); the result is deterministic for a given plan.
 * Errors: EGM_ERR_INVALID_PLAN for a NULL, freed or foreign handle;
 * EGM_ERR_INVALID_VALUE for a missing or unexpected aux, D or operand;
 * EGM_ERR_WORKSPACE; EGM_ERR_ALIGNMENT; EGM_ERR_HIP if a launch fails;
 * EGM_ERR_NOT_SUPPORTED for a pending autotune on a capturing stream (see
 * egm_plan_options_t.autotune).  Nothing is enqueued on an error found by the
 * host checks.
 */
egm_status_t egm_execute(egm_plan_t plan, const void* A, const void* B, void* D, void* aux,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * egm_execute_no_alloc - egm_execute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same launches, with the workspace taken from a
 * static scratch array of EGM_NO_ALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on (from the first call on that GPU until the process
 * ends).  It calls no hipMalloc / hipFree and no allocating routine.
 *   A, B, D, aux, stream  as egm_execute; the stream must belong to the
 *         calling thread's current device, whose scratch is used.
 * Errors: as egm_execute, and EGM_ERR_SCRATCH_LIMIT when the plan's
 * egm_plan_workspace_bytes exceeds EGM_NO_ALLOC_SCRATCH_BYTES (nothing is
 * enqueued); EGM_ERR_NOT_SUPPORTED while an autotune is pending (tuning
 * creates events; run one egm_execute first, or plan without autotune);
 * EGM_ERR_INVALID_VALUE if the stream is on another device.
 * Every call on a GPU shares that GPU's scratch, which keeps whatever the last
 * call left there (the kernels write every scratch byte they later read, so
 * nothing needs clearing): calls whose executions overlap in time on one GPU
 * (different streams, or threads) race on it and must be ordered by the
 * caller.  A plan with no workspace (a fused forward plan) touches no scratch.
 */
egm_status_t egm_execute_no_alloc(egm_plan_t plan, const void* A, const void* B, void* D, void* aux,
                                  void* stream);

/*
 * egm_execute_strided - launch amortisation: the plan on `batch` independent
 * problems of its shape in ONE launch ([op-fusion] §一: each extra kernel
 * launch costs fixed overhead that small operators cannot hide).  Problem z
 * (0 <= z < batch) reads A + z*stride_a and B + z*stride_b (strides in
 * operand elements; 0 shares one operand, e.g. a weight), and writes
 * D + z*stride_d (output elements) and aux + z*stride_aux (bytes); a
 * BIAS_RESIDUAL residual advances with stride_d; the bias (bound at plan) is
 * shared.  The plan must be fused; DRELU_BGRAD is not supported (its partial
 * sums are per launch).  A plan whose tile config came from the per-shape
 * choice (not forced, not autotuned) makes that choice again for the whole
 * batch, whose tiles share the CUs; a forced or autotuned config is kept.  batch <= 65535; 0 does nothing.  Every problem's
 * pointers must keep 16-byte alignment, and outputs must not overlap
 * (stride_d >= m*n, stride_aux >= m*n/8 for batch > 1).  No workspace is
 * needed.  Asynchronous and stream-ordered like egm_execute.
 */
egm_status_t egm_execute_strided(egm_plan_t plan, int64_t batch, const void* A, int64_t stride_a, const void* B,
                                 int64_t stride_b, void* D, int64_t stride_d, void* aux, int64_t stride_aux,
                                 void* stream);

/*
 * egm_layernorm - LayerNorm over the rows of x [rows, cols] (row-major, fp16
 * or bf16), the normalisation that follows the FFN down-projection
 * ([op-fusion] §二, formula and the LayerNorm + residual variant):
 *   y[i,j] = (x[i,j] - mean_i) / sqrt(var_i + eps) * gamma[j] + beta[j] (+ residual[i,j])
 * mean_i and var_i (biased: divided by cols) over row i, from one pass over
 * the row with Welford-style merging of partial statistics in fp32; the
 * result is rounded once to dtype.  The residual is added after the affine
 * step; the post-norm form LN(x + r) is the BIAS_RESIDUAL GEMM epilogue
 * followed by this call without a residual.
 *   gamma, beta  [cols] in dtype, or NULL (1 and 0).   residual  [rows, cols] or NULL.
 *   eps          >= 0 (1e-5 is the usual value).
 *   y            [rows, cols] output; may be x itself (in place).
 *   mean, rstd   [rows] fp32 outputs (1 / sqrt(var + eps)), or NULL.
 *   cols a multiple of 8, 8 <= cols <= 32768; rows >= 0 (0 does nothing).
 *   The launch is one grid dimension of 256-thread workgroups, each covering
 *   256 / tpr rows (tpr = 64 threads per row up to 4096 columns, else 256);
 *   a grid dimension holds at most 2^32 - 1 work-items, so rows above
 *   4 * (2^24 - 1) (cols <= 4096) or 2^24 - 1 (wider rows) give
 *   EGM_ERR_NOT_SUPPORTED.
 * Device pointers 16-byte aligned (mean, rstd 4-byte).  One launch on the
 * stream, asynchronous; no workspace.  Does not need a plan.
 */
egm_status_t egm_layernorm(int64_t rows, int64_t cols, egm_dtype_t dtype, const void* x, const void* residual,
                           const void* gamma, const void* beta, float eps, void* y, float* mean, float* rstd,
                           void* stream);

/* egm_free - release a plan ([bias-fusion] body, checklist: free() releases
 * the plan's resources).  NULL is accepted (EGM_OK).  Handles are never
 * reused: after egm_free, the handle gives EGM_ERR_INVALID_PLAN in every call,
 * a second egm_free included.  Work already enqueued is unaffected; a call of
 * the same plan still running in another thread finishes with the plan. */
egm_status_t egm_free(egm_plan_t plan);

/* Bytes of workspace egm_execute needs for this plan (0 if the handle is NULL,
 * freed or foreign).  The workspace is the caller-owned scratch that stands in
 * for the memory the library would otherwise allocate: the two-kernel path's
 * intermediate product ([bias-fusion] body: the unfused form's extra global
 * write and read) and the bias gradient's per-tile partial sums. */
size_t egm_plan_workspace_bytes(egm_plan_t plan);

/* Write a one-line description of the chosen configuration into buf (always
 * NUL-terminated when len > 0) ([bindings] checklist item 3: inspect the
 * algorithm choice).  EGM_LOG=1 in the environment also prints it at plan time. */
egm_status_t egm_plan_describe(egm_plan_t plan, char* buf, size_t len);

/* Tile-config id the plan will launch (after autotune, the chosen one), or -1
 * for a NULL, freed or foreign handle ([bindings] body, checklist item 3: the
 * algorithm choice can be inspected). */
int32_t egm_plan_config(egm_plan_t plan);

/* Number of tile configurations, and a description of one of them (the
 * candidates plan() chooses among: [bindings] body, checklist item 2).
 * egm_config_describe gives EGM_ERR_INVALID_VALUE for an unknown id or an
 * empty buffer; the text is always NUL-terminated when len > 0. */
int32_t egm_num_configs(void);
egm_status_t egm_config_describe(int32_t config, char* buf, size_t len);

/* Static text for a status code, any int32_t value (never NULL); the pages'
 * interface reports failures as errors ([bias-fusion] body, checklist: a dtype
 * mismatch or a bad bias shape is an error), which this C interface returns
 * as the status codes above. */
const char* egm_status_string(egm_status_t status);

/* EGM_ABI_VERSION of the built library (a caller compares it with the header
 * it was compiled against). */
int32_t egm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EGM_H_ */
