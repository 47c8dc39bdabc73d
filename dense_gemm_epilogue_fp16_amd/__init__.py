"""Python binding of libegm, the fused dense GEMM + epilogue library for MI355X.

Argument marshalling only: every step of D = epilogue(A.B) runs in the HIP
kernels of ``libegm.so`` behind the C ABI of ``include/egm.h``.  PyTorch
supplies device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``); there is no other compute path
and no fallback: if the library is missing, importing this package fails.

Two layers:
  * ``egm_plan`` / ``egm_execute`` / ``egm_free`` / ... : the C functions with
    the same names, on raw integers (device pointers, sizes, a stream handle);
  * ``Matmul``: the stateful object of the bias-fusion page
    ("通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能",
    body, code example): construct with the operands, ``plan(epilog=...,
    epilog_inputs={"bias": ..., "residual": ...})``, ``execute()``, ``free()``,
    usable as a context manager.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# EGM_LIBRARY names another build of the same library (the tests load the
# host-sanitized one this way); there is no other compute path
LIB_PATH = os.environ.get("EGM_LIBRARY") or os.path.join(HERE, "libegm.so")

# status codes (egm_status_t)
EGM_OK = 0
EGM_ERR_INVALID_VALUE = 1
EGM_ERR_NOT_SUPPORTED = 2
EGM_ERR_SHAPE = 3
EGM_ERR_DTYPE = 4
EGM_ERR_ALIGNMENT = 5
EGM_ERR_INVALID_PLAN = 6
EGM_ERR_HIP = 7
EGM_ERR_NO_MEMORY = 8
EGM_ERR_WORKSPACE = 9
EGM_ERR_SCRATCH_LIMIT = 10

#: bytes of the static scratch behind egm_execute_no_alloc (per GPU)
EGM_NO_ALLOC_SCRATCH_BYTES = 32 << 20

# dtypes (egm_dtype_t)
EGM_F16 = 0
EGM_BF16 = 1

# fp8 operand formats (egm_fp8_format_t)
EGM_E4M3 = 0
EGM_E5M2 = 1

# epilogues (egm_epilog_t)
EPILOGS = {
    "DEFAULT": 0,
    "BIAS": 1,
    "RELU_BIAS": 2,
    "GELU_BIAS": 3,
    "RELU_AUX_BIAS": 4,
    "BIAS_RESIDUAL": 5,
    "DRELU": 6,
    "DRELU_BGRAD": 7,
}
BACKWARD_EPILOGS = ("DRELU", "DRELU_BGRAD")

# bias layouts (egm_bias_layout_t)
EGM_BIAS_NONE = 0
EGM_BIAS_ROW = 1  # shape (m, 1)
EGM_BIAS_COL = 2  # shape (1, n)

#: every symbol include/egm.h declares
EXPORTS = (
    "egm_plan", "egm_plan_fp8", "egm_execute", "egm_execute_no_alloc", "egm_execute_strided", "egm_layernorm",
    "egm_free",
    "egm_plan_workspace_bytes",
    "egm_plan_describe",
    "egm_plan_config", "egm_num_configs", "egm_config_describe", "egm_status_string", "egm_abi_version",
)


class EgmError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class EpilogInputs(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("bias_layout", ctypes.c_int32), ("residual", ctypes.c_void_p),
                ("bias_grad", ctypes.c_void_p)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("fused", ctypes.c_int32), ("force_config", ctypes.c_int32),
                ("autotune", ctypes.c_int32), ("group_m", ctypes.c_int32), ("b_transposed", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python dense_gemm_epilogue_fp16_amd/build.py` "
            "(or __graft_entry__.build()); there is no fallback path")
    # torch first, so the library binds to the HIP runtime torch already loaded
    try:
        import torch  # noqa: F401
    except Exception:  # pragma: no cover - torch is part of the environment
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.egm_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, ctypes.POINTER(EpilogInputs),
                             ctypes.POINTER(PlanOptions)]
    lib.egm_plan.restype = i32
    lib.egm_plan_fp8.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, vp, vp, i32,
                                 ctypes.POINTER(EpilogInputs), ctypes.POINTER(PlanOptions)]
    lib.egm_plan_fp8.restype = i32
    lib.egm_execute.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
    lib.egm_execute.restype = i32
    lib.egm_execute_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.egm_execute_no_alloc.restype = i32
    lib.egm_execute_strided.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.egm_execute_strided.restype = i32
    lib.egm_layernorm.argtypes = [i64, i64, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
    lib.egm_layernorm.restype = i32
    lib.egm_free.argtypes = [vp]
    lib.egm_free.restype = i32
    lib.egm_plan_workspace_bytes.argtypes = [vp]
    lib.egm_plan_workspace_bytes.restype = sz
    lib.egm_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
    lib.egm_plan_describe.restype = i32
    lib.egm_plan_config.argtypes = [vp]
    lib.egm_plan_config.restype = i32
    lib.egm_num_configs.argtypes = []
    lib.egm_num_configs.restype = i32
    lib.egm_config_describe.argtypes = [i32, ctypes.c_char_p, sz]
    lib.egm_config_describe.restype = i32
    lib.egm_status_string.argtypes = [i32]
    lib.egm_status_string.restype = ctypes.c_char_p
    lib.egm_abi_version.argtypes = []
    lib.egm_abi_version.restype = i32
    return lib


LIB = _load()
_EXECUTE = LIB.egm_execute


# ---------------------------------------------------------------------------
# the C functions, one to one
# ---------------------------------------------------------------------------
def status_string(status: int) -> str:
    return LIB.egm_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != EGM_OK:
        raise EgmError(status, where)


def egm_plan(m: int, n: int, k: int, dtype: int, epilog: int, bias: int = 0, bias_layout: int = EGM_BIAS_NONE,
             residual: int = 0, *, bias_grad: int = 0, fused: int = 1, force_config: int = -1, autotune: int = 0,
             group_m: int = 0, b_transposed: int = 0, raw_status: bool = False):
    """Returns the plan handle (int), or (status, handle) with ``raw_status``."""
    h = ctypes.c_void_p()
    ins = EpilogInputs(bias or None, bias_layout, residual or None, bias_grad or None)
    opt = PlanOptions(fused, force_config, autotune, group_m, b_transposed)
    st = LIB.egm_plan(ctypes.byref(h), int(m), int(n), int(k), int(dtype), int(epilog), ctypes.byref(ins),
                      ctypes.byref(opt))
    if raw_status:
        return st, h.value
    _check(st, "egm_plan")
    return h.value


def egm_plan_fp8(m: int, n: int, k: int, a_format: int, b_format: int, out_dtype: int, scale_a: int, scale_b: int,
                 epilog: int, bias: int = 0, bias_layout: int = EGM_BIAS_NONE, residual: int = 0, *, fused: int = 1,
                 force_config: int = -1, autotune: int = 0, group_m: int = 0, b_transposed: int = 0,
                 raw_status: bool = False):
    """fp8 operands with per-tensor scales (device pointers to one fp32 each,
    0 = NULL = 1); returns the plan handle, or (status, handle) with ``raw_status``."""
    h = ctypes.c_void_p()
    ins = EpilogInputs(bias or None, bias_layout, residual or None, None)
    opt = PlanOptions(fused, force_config, autotune, group_m, b_transposed)
    st = LIB.egm_plan_fp8(ctypes.byref(h), int(m), int(n), int(k), int(a_format), int(b_format), int(out_dtype),
                          scale_a or None, scale_b or None, int(epilog), ctypes.byref(ins), ctypes.byref(opt))
    if raw_status:
        return st, h.value
    _check(st, "egm_plan_fp8")
    return h.value


def egm_execute(plan: int, A: int, B: int, D: int, aux: int = 0, workspace: int = 0, workspace_bytes: int = 0,
                stream: int = 0, raw_status: bool = False):
    st = LIB.egm_execute(plan, A or None, B or None, D or None, aux or None, workspace or None,
                         int(workspace_bytes), stream or None)
    if raw_status:
        return st
    _check(st, "egm_execute")
    return None


def egm_execute_no_alloc(plan: int, A: int, B: int, D: int, aux: int = 0, stream: int = 0,
                         raw_status: bool = False):
    """egm_execute with the library's static scratch as the workspace (no
    device allocation anywhere on the call)."""
    st = LIB.egm_execute_no_alloc(plan, A or None, B or None, D or None, aux or None, stream or None)
    if raw_status:
        return st
    _check(st, "egm_execute_no_alloc")
    return None


def egm_execute_strided(plan: int, batch: int, A: int, stride_a: int, B: int, stride_b: int, D: int, stride_d: int,
                        aux: int = 0, stride_aux: int = 0, stream: int = 0, raw_status: bool = False):
    st = LIB.egm_execute_strided(plan, int(batch), A or None, int(stride_a), B or None, int(stride_b), D or None,
                                 int(stride_d), aux or None, int(stride_aux), stream or None)
    if raw_status:
        return st
    _check(st, "egm_execute_strided")
    return None


def egm_layernorm(rows: int, cols: int, dtype: int, x: int, residual: int, gamma: int, beta: int, eps: float,
                  y: int, mean: int = 0, rstd: int = 0, stream: int = 0, raw_status: bool = False):
    st = LIB.egm_layernorm(int(rows), int(cols), int(dtype), x or None, residual or None, gamma or None,
                           beta or None, float(eps), y or None, mean or None, rstd or None, stream or None)
    if raw_status:
        return st
    _check(st, "egm_layernorm")
    return None


def layer_norm(x, gamma=None, beta=None, eps: float = 1e-5, residual=None, out=None, return_stats: bool = False,
               stream=None):
    """LayerNorm over the last axis of a 2-D fp16/bf16 GPU tensor x [rows, cols]:
    (x - mean) / sqrt(var + eps) * gamma + beta (+ residual), one launch of the
    library's row kernel.  ``out`` may be x (in place).  With ``return_stats``
    also returns the fp32 mean and rstd per row."""
    import torch
    for t, name in ((x, "x"), (residual, "residual"), (out, "out")):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype or tuple(t.shape) !=
                              tuple(x.shape) or t.dim() != 2):
            raise ValueError(f"{name} must be a contiguous [rows, cols] GPU tensor in x's dtype")
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype or t.numel() != x.shape[1]):
            raise ValueError(f"{name} must be a contiguous [cols] GPU tensor in x's dtype")
    rows, cols = x.shape
    y = out if out is not None else torch.empty_like(x)
    mean = rstd = None
    if return_stats:
        mean = torch.empty(rows, dtype=torch.float32, device=x.device)
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    egm_layernorm(rows, cols, _dtype_code(x), x.data_ptr(), residual.data_ptr() if residual is not None else 0,
                  gamma.data_ptr() if gamma is not None else 0, beta.data_ptr() if beta is not None else 0, eps,
                  y.data_ptr(), mean.data_ptr() if mean is not None else 0,
                  rstd.data_ptr() if rstd is not None else 0, s.cuda_stream)
    return (y, mean, rstd) if return_stats else y


def egm_free(plan: int, raw_status: bool = False):
    st = LIB.egm_free(plan)
    if raw_status:
        return st
    _check(st, "egm_free")
    return None


def egm_plan_workspace_bytes(plan: int) -> int:
    return int(LIB.egm_plan_workspace_bytes(plan))


def egm_plan_describe(plan: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(LIB.egm_plan_describe(plan, buf, len(buf)), "egm_plan_describe")
    return buf.value.decode()


def egm_plan_config(plan: int) -> int:
    return int(LIB.egm_plan_config(plan))


def egm_num_configs() -> int:
    return int(LIB.egm_num_configs())


def egm_config_describe(config: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(LIB.egm_config_describe(int(config), buf, len(buf)), "egm_config_describe")
    return buf.value.decode()


def egm_abi_version() -> int:
    return int(LIB.egm_abi_version())


# ---------------------------------------------------------------------------
# torch-facing stateful object
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.float16:
        return EGM_F16
    if dt == torch.bfloat16:
        return EGM_BF16
    raise TypeError(f"dtype {dt} not supported: fp16 or bf16 only")


def _is_transposed_view(t) -> bool:
    """True for a 2-D tensor that is the transpose of a contiguous one
    (strides (1, rows)), e.g. w.t() for a contiguous w; not for a tensor that
    is also contiguous (a single row or column)."""
    return t.dim() == 2 and not t.is_contiguous() and t.stride() == (1, t.shape[0])


def _fp8_code(t):
    """egm_fp8_format_t of an fp8 tensor (OCP float8_e4m3fn / float8_e5m2), else None."""
    import torch
    if t.dtype == torch.float8_e4m3fn:
        return EGM_E4M3
    if t.dtype == torch.float8_e5m2:
        return EGM_E5M2
    return None


class Matmul:
    """D = epilogue(a @ b) for row-major a [m,k], b [k,n] torch tensors on the GPU.

    ``plan(epilog="BIAS", epilog_inputs={"bias": t})`` with ``t`` shaped
    (m,1) or (1,n) (any other shape is rejected); ``"residual"`` [m,n] for
    BIAS_RESIDUAL.  ``execute()`` enqueues on torch's current stream and
    returns D (and the packed [m, n/8] uint8 mask for RELU_AUX_BIAS).
    ``a`` and ``b`` may be rebound per call: ``execute(a=..., b=...)``.

    Backward: ``plan("DRELU")`` and ``plan("DRELU_BGRAD", {"bias_grad": g})``
    with ``g`` a float32 tensor shaped (m,1) (gradient of an (m,1) bias: row
    sums) or (1,n) (of a (1,n) bias: column sums); ``execute(aux=mask)`` takes
    the forward RELU_AUX_BIAS mask as input and returns D (and ``g``).

    fp8: ``a`` and ``b`` of dtype float8_e4m3fn / float8_e5m2 (any pairing),
    ``scale_a`` / ``scale_b`` one-element float32 GPU tensors (None = 1),
    ``out_dtype`` fp16 or bf16 (default bf16) for D, the bias and the residual.

    ``b`` may be a transposed view of a contiguous [n, k] tensor (``w.t()``,
    a linear layer's weight): the plan then reads it in that layout, with no
    copy (the ``b_transposed`` plan option).

    ``execute(stream=s)`` launches on ``s`` and allocates the outputs there.
    The two-kernel path and DRELU_BGRAD use a workspace that the plan
    allocates once and every execute of that plan shares: such executes must
    not overlap in time (keep them on one stream, or order the streams).
    """

    def __init__(self, a, b, *, scale_a=None, scale_b=None, out_dtype=None):
        import torch
        fa, fb = _fp8_code(a), _fp8_code(b)
        self.fp8 = None
        if fa is not None or fb is not None:
            if fa is None or fb is None:
                raise TypeError("fp8 operands come in pairs (no implicit conversion)")
            self.fp8 = (fa, fb)
            out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
            _dtype_code(out_dtype)
            for t, name in ((scale_a, "scale_a"), (scale_b, "scale_b")):
                if t is not None and (not t.is_cuda or t.dtype != torch.float32 or t.numel() != 1):
                    raise ValueError(f"{name} must be a one-element float32 GPU tensor")
        else:
            if scale_a is not None or scale_b is not None:
                raise ValueError("scales belong to fp8 operands")
            if out_dtype is not None and out_dtype != a.dtype:
                raise TypeError("16-bit operands produce their own dtype (no implicit conversion)")
            out_dtype = a.dtype
        self.bt = _is_transposed_view(b)
        self._check_operand(a, "a", fp8=self.fp8 is not None)
        self._check_operand(b, "b", fp8=self.fp8 is not None, transposed=self.bt)
        if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
            raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not multiply")
        if self.fp8 is None and a.dtype != b.dtype:
            raise TypeError("a and b must share one dtype (no implicit conversion)")
        self.a, self.b = a, b
        self._dev = a.device.index if a.device.index is not None else torch.cuda.current_device()
        self.scale_a, self.scale_b = scale_a, scale_b
        self.m, self.k = a.shape
        self.n = b.shape[1]
        self.dtype = out_dtype
        self._plan = None
        self._keep = ()
        self._res_batch = 0
        self.epilog = None

    @staticmethod
    def _check_operand(t, name, fp8=False, transposed=False):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if transposed:
            if not _is_transposed_view(t):
                raise ValueError(f"{name} must be a transposed view of a contiguous tensor, as planned")
        elif not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous row-major (or, for b, a transposed contiguous tensor)")
        if fp8:
            if _fp8_code(t) is None:
                raise TypeError(f"{name}: dtype {t.dtype} is not an fp8 operand type")
        else:
            _dtype_code(t)

    def plan(self, epilog: str = "DEFAULT", epilog_inputs: dict | None = None, *, fused: bool = True,
             force_config: int = -1, autotune: bool = False, group_m: int = 0):
        if epilog not in EPILOGS:
            raise ValueError(f"unknown epilog {epilog!r}; one of {sorted(EPILOGS)}")
        ins = dict(epilog_inputs or {})
        unknown = set(ins) - {"bias", "residual", "bias_grad"}
        if unknown:
            raise ValueError(f"unknown epilog inputs {sorted(unknown)}")
        bias_ptr, layout, res_ptr, grad_ptr = 0, EGM_BIAS_NONE, 0, 0
        keep = []
        self.bias_grad = None
        if "bias_grad" in ins:
            import torch
            g = ins["bias_grad"]
            if not g.is_cuda or not g.is_contiguous() or g.dtype != torch.float32:
                raise ValueError("bias_grad must be a contiguous float32 GPU tensor")
            if tuple(g.shape) == (self.m, 1):
                layout = EGM_BIAS_ROW
            elif tuple(g.shape) == (1, self.n):
                layout = EGM_BIAS_COL
            else:
                raise ValueError(f"bias_grad shape {tuple(g.shape)} must be (m,1)=({self.m},1) or (1,n)=(1,{self.n})")
            grad_ptr = g.data_ptr()
            keep.append(g)
            self.bias_grad = g
        if "bias" in ins:
            bias = ins["bias"]
            self._check_operand(bias, "bias")
            if bias.dtype != self.dtype:
                raise TypeError("bias dtype must match a and b (no implicit conversion)")
            if tuple(bias.shape) == (self.m, 1):
                layout = EGM_BIAS_ROW
            elif tuple(bias.shape) == (1, self.n):
                layout = EGM_BIAS_COL
            else:
                raise ValueError(f"bias shape {tuple(bias.shape)} must be (m,1)=({self.m},1) or (1,n)=(1,{self.n})")
            bias_ptr = bias.data_ptr()
            keep.append(bias)
        self._res_batch = 0
        if "residual" in ins:
            r = ins["residual"]
            self._check_operand(r, "residual")
            if r.dtype != self.dtype or tuple(r.shape[-2:]) != (self.m, self.n) or r.dim() not in (2, 3):
                raise ValueError("residual must be [m,n] (or [batch,m,n] for execute_batched) in the output dtype")
            self._res_batch = r.shape[0] if r.dim() == 3 else 1
            res_ptr = r.data_ptr()
            keep.append(r)
        self.free()
        if self.fp8 is not None:
            if grad_ptr:
                raise ValueError("the backward epilogues take 16-bit operands")
            sa = self.scale_a.data_ptr() if self.scale_a is not None else 0
            sb = self.scale_b.data_ptr() if self.scale_b is not None else 0
            keep += [t for t in (self.scale_a, self.scale_b) if t is not None]
            self._plan = egm_plan_fp8(self.m, self.n, self.k, self.fp8[0], self.fp8[1], _dtype_code(self.dtype), sa,
                                      sb, EPILOGS[epilog], bias_ptr, layout, res_ptr, fused=int(fused),
                                      force_config=force_config, autotune=int(autotune), group_m=group_m,
                                      b_transposed=int(self.bt))
        else:
            self._plan = egm_plan(self.m, self.n, self.k, _dtype_code(self.a), EPILOGS[epilog], bias_ptr, layout,
                                  res_ptr, bias_grad=grad_ptr, fused=int(fused), force_config=force_config,
                                  autotune=int(autotune), group_m=group_m, b_transposed=int(self.bt))
        self._keep = tuple(keep)
        self.epilog = epilog
        self._ws = None
        wsb = egm_plan_workspace_bytes(self._plan)
        if wsb:
            import torch
            self._ws = torch.empty(wsb, dtype=torch.uint8, device=self.a.device)
        return self

    def describe(self) -> str:
        return egm_plan_describe(self._require())

    def _require(self):
        if self._plan is None:
            raise RuntimeError("call plan() first")
        return self._plan

    def execute(self, a=None, b=None, out=None, aux=None, stream=None):
        import torch
        plan = self._require()
        # the planned operands need no re-check; rebound ones keep shape and dtype
        if a is None:
            a = self.a
        elif a is not self.a:
            self._check_rebound(a, (self.m, self.k), self.a.dtype)
        if b is None:
            b = self.b
        elif b is not self.b:
            self._check_rebound(b, (self.k, self.n), self.b.dtype, transposed=self.bt)
        if out is None:
            d = self._new((self.m, self.n), self.dtype, a.device, stream)
        else:
            self._check_output(out, (self.m, self.n), self.dtype, "out")
            d = out
        mask = None
        if self.epilog == "RELU_AUX_BIAS":
            if aux is None:
                mask = self._new((self.m, self.n // 8), torch.uint8, a.device, stream)
            else:
                self._check_output(aux, (self.m, self.n // 8), torch.uint8, "aux")
                mask = aux
        elif self.epilog in BACKWARD_EPILOGS:
            if aux is None:
                raise ValueError("the backward epilogues take the forward mask: aux = uint8 [m, n/8] on the GPU")
            self._check_output(aux, (self.m, self.n // 8), torch.uint8, "aux")
            mask = aux
        elif aux is not None:
            raise ValueError(f"{self.epilog} takes no mask")
        raw = stream.cuda_stream if stream is not None else torch._C._cuda_getCurrentRawStream(self._dev)
        ws = self._ws
        if ws is not None and stream is not None:
            ws.record_stream(stream)  # the allocator must not reuse it before this launch ends
        st = _EXECUTE(plan, a.data_ptr(), b.data_ptr(), d.data_ptr(), mask.data_ptr() if mask is not None else None,
                      ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, raw)
        if st != EGM_OK:
            raise EgmError(st, "egm_execute")
        if self.epilog == "DRELU_BGRAD":
            return d, self.bias_grad
        if self.epilog == "DRELU":
            return d
        return (d, mask) if mask is not None else d

    @staticmethod
    def _new(shape, dtype, device, stream):
        # outputs belong to the stream the launch runs on, as torch's own ops do
        import torch
        if stream is None:
            return torch.empty(shape, dtype=dtype, device=device)
        with torch.cuda.stream(stream):
            return torch.empty(shape, dtype=dtype, device=device)

    def _check_rebound(self, t, shape, dtype, transposed=False):
        self._check_operand(t, "operand", fp8=self.fp8 is not None, transposed=transposed)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError("rebound operand must keep the planned shape and dtype")

    @staticmethod
    def _check_output(t, shape, dtype, name):
        if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {shape}")

    def execute_batched(self, a, b, out=None, aux=None, stream=None):
        """One launch over a batch of problems of the planned shape: ``a`` is
        [batch, m, k] or the planned [m, k] shared by every problem, ``b`` is
        [batch, k, n] or [k, n] shared; returns D [batch, m, n] (and the
        [batch, m, n/8] mask for RELU_AUX_BIAS).  DRELU takes ``aux`` as the
        [batch, m, n/8] input mask.  A BIAS_RESIDUAL residual bound at plan
        must then be [batch, m, n].  Every problem's buffers must start
        16-byte aligned: with masks, m*n/8 must be a multiple of 16."""
        import torch
        plan = self._require()
        batch = None
        strides = []
        for t, shape, dt, tr in ((a, (self.m, self.k), self.a.dtype, False),
                                 (b, (self.k, self.n), self.b.dtype, self.bt)):
            if not t.is_cuda or t.dtype != dt:
                raise ValueError("batched operands are GPU tensors of the planned dtype")
            if tuple(t.shape) == shape:
                self._check_operand(t, "operand", fp8=self.fp8 is not None, transposed=tr)
                strides.append(0)
            elif t.dim() == 3 and tuple(t.shape[1:]) == shape:
                # each problem's matrix in the planned layout, problems back to back
                want = (shape[0] * shape[1], 1, shape[0]) if tr else (shape[0] * shape[1], shape[1], 1)
                if t.stride() != want:
                    raise ValueError(f"batched operand strides {t.stride()} must be {want}")
                if batch is not None and t.shape[0] != batch:
                    raise ValueError("batch sizes differ")
                batch = t.shape[0]
                strides.append(shape[0] * shape[1])
            else:
                raise ValueError(f"operand shape {tuple(t.shape)} is neither {shape} nor [batch, *{shape}]")
        if batch is None:
            raise ValueError("at least one operand must carry the batch dimension")
        if self.epilog == "BIAS_RESIDUAL" and self._res_batch < batch:
            raise ValueError(f"the residual bound at plan holds {self._res_batch} problems, the batch {batch}: it "
                             "advances with D and must be [batch, m, n]")
        if out is not None:
            self._check_output(out, (batch, self.m, self.n), self.dtype, "out")
        d = out if out is not None else self._new((batch, self.m, self.n), self.dtype, a.device, stream)
        mask = None
        if self.epilog == "RELU_AUX_BIAS":
            if aux is not None:
                self._check_output(aux, (batch, self.m, self.n // 8), torch.uint8, "aux")
            mask = aux if aux is not None else self._new((batch, self.m, self.n // 8), torch.uint8, a.device, stream)
        elif self.epilog == "DRELU":
            if aux is None:
                raise ValueError("DRELU takes the forward masks: aux = uint8 [batch, m, n/8] on the GPU")
            self._check_output(aux, (batch, self.m, self.n // 8), torch.uint8, "aux")
            mask = aux
        elif aux is not None:
            raise ValueError(f"{self.epilog} takes no mask")
        s = stream if stream is not None else torch.cuda.current_stream(a.device)
        egm_execute_strided(plan, batch, a.data_ptr(), strides[0], b.data_ptr(), strides[1], d.data_ptr(),
                            self.m * self.n, mask.data_ptr() if mask is not None else 0,
                            self.m * (self.n // 8) if mask is not None else 0, s.cuda_stream)
        return (d, mask) if self.epilog == "RELU_AUX_BIAS" else d

    def free(self):
        if self._plan is not None:
            egm_free(self._plan)
            self._plan = None
            self._keep = ()
            self._ws = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()
        return False

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
