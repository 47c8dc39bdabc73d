"""CPU fp64 oracle for the fused dense GEMM + epilogue  D = epilogue(A.B).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or run this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``dense_gemm_epilogue_fp16_amd``) and imports nothing from it.

Pages cited (by title, with the part of the page meant):
  [bias-fusion]  "通过 nvmath-python 的 cuBLASLt 绑定，在 PyTorch 中实现偏差融合以提升推理性能"
                 (blog.hotdry.top, 2025-09-22): fusing bias / ReLU into the
                 cuBLASLt GEMM through nvmath-python's stateful Matmul API.
  [bindings]     "nvmath-python：cuBLAS与cuSOLVER的Python绑定加速ML线性代数"
                 (blog.hotdry.top, 2025-09-19).
  [op-fusion]    "模型推理中的算子融合优化从LayerNorm到残差连接的图级优化"
                 (wmrh.cn news 429806): operator fusion for inference.

What is computed (the plain definition; the fused kernel reaches the same
result up to fp32 accumulation order and one final rounding):
  1. P = A.B, every 16-bit operand widened exactly to fp64, summed in fp64.
  2. Z = P + bias, bias broadcast per row (shape (m,1)) or per column (shape
     (1,n)) [bias-fusion, body: shape-constraint item of the checklist].
  3. Y = epilogue(Z): identity (BIAS), max(Z,0) (RELU_BIAS: multiply, add bias,
     then activate [bias-fusion, body, paragraph before the code example]),
     tanh-form GELU (GELU_BIAS [op-fusion §一 FFN chain; bias-fusion, body,
     closing paragraph names GELU as an epilogue]), Z + R (BIAS_RESIDUAL: the
     residual added to the producer's output [op-fusion §三]); DEFAULT is P.
  4. RELU_AUX_BIAS also returns the ReLU mask needed by backward
     [bias-fusion, body, limitations paragraph on training].
Readings where the pages say nothing precise (each is listed in the design
notes): the GELU is the tanh form with sqrt(2/pi) and 0.044715 (Hendrycks &
Gimpel); the mask bit is Z > 0 on the pre-activation after the bias, packed
row-major [m, n/8] uint8, least-significant bit first (bit b of byte c is column
8c+b); bias, residual and output share the operand dtype.

Backward epilogues (the consumers of that mask; [bias-fusion], body: the
training paragraph says the forward pass must leave the mask the backward pass
needs, and the closing paragraph names dBias as an epilogue to come):
  DRELU        dZ = P (.) mask, where P = A.B is the gradient reaching the
               ReLU output and mask is the packed (Z > 0) of the forward pass;
               D = dZ rounded to the operand dtype.
  DRELU_BGRAD  the same, plus the bias gradient: dZ summed over the axis the
               forward bias was broadcast along ((1,n) bias: over rows, n
               values; (m,1) bias: over columns, m values), from the unrounded
               dZ, returned in fp32.

FP8 operands ([bias-fusion], body: the data-type item of the checklist lists
FP8 among the supported types; the closing paragraph names FP8 among the
features to come).  The operands are OCP 8-bit floats, E4M3 (4 exponent bits,
bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN) or E5M2 (5
exponent bits, bias 15, 2 mantissa bits, IEEE-style infinities and NaNs), each
with a per-tensor fp32 dequantisation scale: A = scale_a * A8, B = scale_b *
B8.  The page's same-type rule is read as covering the two operands; the bias,
the residual and the output are 16-bit (fp16 or bf16), since an fp8 bias or
output would lose the precision the epilogue exists to keep.  Then
  Z = scale_a * scale_b * (A8 . B8) + bias,  Y = epilogue(Z)
with the same epilogues as above.

LayerNorm after the down-projection ([op-fusion] §二: the formula
y = (x - mu) / sqrt(sigma^2 + eps) * gamma + beta over the last axis, eps 1e-5
by default, and the variant that adds a residual to the normalised output;
the page computes mean and variance in one pass with Welford's method, which
reaches the same statistics up to rounding): mu is the row mean, sigma^2 the
row's biased variance (divided by the row length), gamma and beta per column.
The oracle is that definition in fp64.

Every function here is pinned by ``tests/test_oracle_pins.py`` against brute
force, closed forms, invariants and library routines.
"""
from __future__ import annotations

import math

import numpy as np

F16 = "fp16"
BF16 = "bf16"

EPILOGS = ("DEFAULT", "BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL")
BACKWARD_EPILOGS = ("DRELU", "DRELU_BGRAD")

# unit roundoff of the fp32 accumulation the GPU path uses
FP32_U = 2.0 ** -24

# tanh-form GELU constants (Hendrycks & Gimpel, "Gaussian Error Linear Units")
GELU_C0 = math.sqrt(2.0 / math.pi)
GELU_C1 = 0.044715

# max |D - Y| allowed per output dtype (fp16 out, bf16 out)
TOLERANCE = {F16: 1e-2, BF16: 2e-2}


# ---------------------------------------------------------------------------
# exact widening of operand bit patterns
# ---------------------------------------------------------------------------
def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16 / bf16 bit patterns (uint16) -> float64, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        # a bf16 value is the upper half of the fp32 with the same pattern
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# step 1: the product
# ---------------------------------------------------------------------------
def product(a64: np.ndarray, b64: np.ndarray) -> np.ndarray:
    """P = A.B in fp64 (a textbook dgemm).  Products of two 16-bit floats are
    exact in fp64; the summation error is below K * 2^-53 * sum|a||b|."""
    a64 = np.asarray(a64, dtype=np.float64)
    b64 = np.asarray(b64, dtype=np.float64)
    if a64.shape[1] == 0:
        return np.zeros((a64.shape[0], b64.shape[1]), dtype=np.float64)
    return a64 @ b64


# ---------------------------------------------------------------------------
# step 2: bias broadcast
# ---------------------------------------------------------------------------
def add_bias(p: np.ndarray, bias64: np.ndarray, layout: str) -> np.ndarray:
    """Z = P + bias; "row" = bias of shape (m,1) added to every column of row i,
    "col" = bias of shape (1,n) added to every row of column j
    [bias-fusion, body: shape-constraint item of the checklist]."""
    bias64 = np.asarray(bias64, dtype=np.float64).reshape(-1)
    if layout == "row":
        if bias64.shape[0] != p.shape[0]:
            raise ValueError("row bias must have m entries")
        return p + bias64[:, None]
    if layout == "col":
        if bias64.shape[0] != p.shape[1]:
            raise ValueError("col bias must have n entries")
        return p + bias64[None, :]
    raise ValueError(f"unknown bias layout {layout!r}")


# ---------------------------------------------------------------------------
# step 3: the activation / residual
# ---------------------------------------------------------------------------
def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(GELU_C0 * (z + GELU_C1 * z * z * z)))


def relu(z: np.ndarray) -> np.ndarray:
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def apply_epilog(z: np.ndarray, epilog: str, r64: np.ndarray | None = None) -> np.ndarray:
    """Y from the pre-activation Z (Z = P for DEFAULT)."""
    if epilog in ("DEFAULT", "BIAS"):
        return np.asarray(z, dtype=np.float64)
    if epilog in ("RELU_BIAS", "RELU_AUX_BIAS"):
        return relu(z)
    if epilog == "GELU_BIAS":
        return gelu_tanh(z)
    if epilog == "BIAS_RESIDUAL":
        if r64 is None:
            raise ValueError("BIAS_RESIDUAL needs the residual")
        return np.asarray(z, dtype=np.float64) + np.asarray(r64, dtype=np.float64)
    raise ValueError(f"unknown epilog {epilog!r}")


# ---------------------------------------------------------------------------
# step 4: the auxiliary ReLU mask
# ---------------------------------------------------------------------------
def relu_mask(z: np.ndarray) -> np.ndarray:
    """Packed (Z > 0): uint8 [m, n/8], bit b of byte c = column 8c+b."""
    z = np.asarray(z, dtype=np.float64)
    if z.shape[1] % 8:
        raise ValueError("n must be a multiple of 8 for the packed mask")
    return np.packbits(z > 0.0, axis=1, bitorder="little")


# ---------------------------------------------------------------------------
# rounding fp64 -> fp16 / bf16 (nearest, ties to even), for ulp statistics and
# for feeding a rounded intermediate into a following GEMM
# ---------------------------------------------------------------------------
_FORMAT = {
    # significand bits (with the implicit one), exponent of the smallest normal,
    # largest finite value
    F16: (11, -14, 65504.0),
    BF16: (8, -126, float.fromhex("0x1.fep127")),
}


def round_to_bits(y: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values once, to nearest-even, to fp16 / bf16; return bits."""
    sig, emin, vmax = _FORMAT[dtype]
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)                      # |y| in [2^(e-1), 2^e)
    lead = np.maximum(e - 1, emin)          # weight of the leading bit (subnormals share emin)
    q = np.ldexp(np.ones_like(y), lead - (sig - 1))  # spacing of representable values
    r = np.round(y / q) * q                 # numpy rounds halves to even; scaling by 2^n is exact
    r = np.where(np.abs(r) > vmax, np.copysign(np.inf, y), r)
    if dtype == F16:
        return r.astype(np.float16).view(np.uint16)          # exact: r is representable
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def ulp(y: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit format at |y| (for the double-rounding bound): the
    gap above the binade |y| lies in; zero and the subnormals share the
    subnormal spacing 2^(emin - (sig - 1))."""
    sig, emin, _ = _FORMAT[dtype]
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)                      # |y| in [2^(e-1), 2^e); frexp(0) gives e = 0
    lead = np.where(y == 0.0, emin, np.maximum(e - 1, emin))
    return np.ldexp(1.0, lead - (sig - 1))


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------
def reference(a_bits, b_bits, dtype, epilog, bias_bits=None, bias_layout=None,
              residual_bits=None, rows=None):
    """Unrounded Y (fp64), pre-activation Z (fp64) and, for RELU_AUX_BIAS, the
    packed mask.  ``rows`` restricts the computation to those output rows (the
    row bias, the residual and A are sliced to match)."""
    if epilog not in EPILOGS:
        raise ValueError(f"unknown epilog {epilog!r}")
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    r_bits = None if residual_bits is None else np.asarray(residual_bits, dtype=np.uint16)
    row_bias = bias_bits
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        a_bits = a_bits[rows]
        if r_bits is not None:
            r_bits = r_bits[rows]
        if bias_layout == "row" and bias_bits is not None:
            row_bias = np.asarray(bias_bits, dtype=np.uint16).reshape(-1)[rows]
    z = product(widen(a_bits, dtype), widen(b_bits, dtype))
    if epilog != "DEFAULT":
        if bias_bits is None or bias_layout is None:
            raise ValueError(f"{epilog} needs a bias")
        z = add_bias(z, widen(row_bias, dtype), bias_layout)
    r64 = widen(r_bits, dtype) if r_bits is not None else None
    y = apply_epilog(z, epilog, r64)
    mask = relu_mask(z) if epilog == "RELU_AUX_BIAS" else None
    return y, z, mask


# ---------------------------------------------------------------------------
# fp8 operands: exact decoding and the scaled product
# ---------------------------------------------------------------------------
E4M3 = "e4m3"
E5M2 = "e5m2"
# exponent bits, mantissa bits, exponent bias
FP8_FORMATS = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}


def decode_fp8(bits: np.ndarray, fmt: str) -> np.ndarray:
    """fp8 bit patterns (uint8) -> float64, exactly, from the bit fields:
    a normal number (exponent field e > 0) is (-1)^s 2^(e - bias) (1 + m 2^-M),
    a subnormal one (e = 0) is (-1)^s 2^(1 - bias) m 2^-M.  E4M3 spends only
    its all-ones pattern (e and m all ones) on NaN and has no infinities; E5M2
    keeps the IEEE convention for an all-ones exponent (m = 0: infinity, else
    NaN)."""
    if fmt not in FP8_FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    ebits, mbits, bias = FP8_FORMATS[fmt]
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = b >> 7
    e = (b >> mbits) & ((1 << ebits) - 1)
    m = b & ((1 << mbits) - 1)
    normal = np.ldexp((m + (1 << mbits)).astype(np.float64), e - bias - mbits)
    subnormal = np.ldexp(m.astype(np.float64), 1 - bias - mbits)
    mag = np.where(e == 0, subnormal, normal)
    top = (1 << ebits) - 1
    if fmt == E4M3:
        mag = np.where((e == top) & (m == (1 << mbits) - 1), np.nan, mag)
    else:
        mag = np.where(e == top, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(sign == 1, -mag, mag)


def reference_fp8(a_bits, b_bits, a_fmt, b_fmt, scale_a, scale_b, out_dtype, epilog, bias_bits=None,
                  bias_layout=None, residual_bits=None, rows=None):
    """Y, Z and the mask (as ``reference``) for fp8 operands with per-tensor
    fp32 scales: Z = scale_a scale_b (A8 . B8) + bias.  Products of two fp8
    values are exact in fp64; the two fp32 scales multiply exactly in fp64.
    bias_bits and residual_bits are in the 16-bit out_dtype."""
    if epilog not in EPILOGS:
        raise ValueError(f"unknown epilog {epilog!r}")
    a_bits = np.asarray(a_bits, dtype=np.uint8)
    r_bits = None if residual_bits is None else np.asarray(residual_bits, dtype=np.uint16)
    row_bias = bias_bits
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        a_bits = a_bits[rows]
        if r_bits is not None:
            r_bits = r_bits[rows]
        if bias_layout == "row" and bias_bits is not None:
            row_bias = np.asarray(bias_bits, dtype=np.uint16).reshape(-1)[rows]
    scale = float(np.float32(scale_a)) * float(np.float32(scale_b))
    z = product(decode_fp8(a_bits, a_fmt), decode_fp8(b_bits, b_fmt)) * scale
    if epilog != "DEFAULT":
        if bias_bits is None or bias_layout is None:
            raise ValueError(f"{epilog} needs a bias")
        z = add_bias(z, widen(row_bias, out_dtype), bias_layout)
    r64 = widen(r_bits, out_dtype) if r_bits is not None else None
    y = apply_epilog(z, epilog, r64)
    mask = relu_mask(z) if epilog == "RELU_AUX_BIAS" else None
    return y, z, mask


# ---------------------------------------------------------------------------
# backward: the ReLU mask applied to an incoming gradient, and the bias gradient
# ---------------------------------------------------------------------------
def unpack_mask(mask: np.ndarray, n: int) -> np.ndarray:
    """Packed uint8 [m, n/8] (bit b of byte c = column 8c+b) -> bool [m, n]."""
    mask = np.asarray(mask, dtype=np.uint8)
    if mask.shape[1] * 8 != n:
        raise ValueError("mask must hold n/8 bytes per row")
    return np.unpackbits(mask, axis=1, bitorder="little").astype(bool)


def drelu(p: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """dZ = dY (.) 1[Z > 0]: the gradient P = A.B reaching the ReLU output,
    kept where the forward pre-activation was positive."""
    p = np.asarray(p, dtype=np.float64)
    return np.where(unpack_mask(mask, p.shape[1]), p, 0.0)


def bias_grad(dz: np.ndarray, layout: str) -> np.ndarray:
    """Gradient of a broadcast bias: a (1,n) bias ("col") collects the sum over
    rows, an (m,1) bias ("row") the sum over columns."""
    dz = np.asarray(dz, dtype=np.float64)
    if layout == "col":
        return dz.sum(axis=0)
    if layout == "row":
        return dz.sum(axis=1)
    raise ValueError(f"unknown bias layout {layout!r}")


def bias_grad_error_bound(a64: np.ndarray, b64: np.ndarray, mask: np.ndarray, layout: str) -> np.ndarray:
    """Worst-case error of a bias gradient accumulated in fp32: every dZ value
    carries at most K u (|A|.|B|)_ij from its K-term fp32 dot product, and the
    L-term fp32 sum along the reduced axis adds at most L u sum|dZ|, so the
    total stays below (K + L) u sum over the reduced axis of (|A|.|B|) (.) mask
    (first-order bound, u = 2^-24)."""
    absprod = product(np.abs(np.asarray(a64, dtype=np.float64)), np.abs(np.asarray(b64, dtype=np.float64)))
    kept = np.where(unpack_mask(mask, absprod.shape[1]), absprod, 0.0)
    k = np.asarray(a64).shape[1]
    reduced_len = kept.shape[0] if layout == "col" else kept.shape[1]
    return (k + reduced_len) * FP32_U * bias_grad(kept, layout)


def backward_reference(a_bits, b_bits, dtype, epilog, mask, bias_layout=None):
    """Unrounded dZ (fp64), and for DRELU_BGRAD the bias gradient (fp64) with
    its fp32-accumulation error bound."""
    if epilog not in BACKWARD_EPILOGS:
        raise ValueError(f"unknown backward epilog {epilog!r}")
    a64 = widen(a_bits, dtype)
    b64 = widen(b_bits, dtype)
    dz = drelu(product(a64, b64), mask)
    if epilog == "DRELU":
        return dz, None, None
    if bias_layout is None:
        raise ValueError("DRELU_BGRAD needs the bias layout")
    return dz, bias_grad(dz, bias_layout), bias_grad_error_bound(a64, b64, mask, bias_layout)


# ---------------------------------------------------------------------------
# LayerNorm over the last axis ([op-fusion] §二)
# ---------------------------------------------------------------------------
LN_EPS = 1e-5


def layer_norm(x64: np.ndarray, gamma64=None, beta64=None, eps: float = LN_EPS, r64=None):
    """y = (x - mean) / sqrt(var + eps) * gamma + beta (+ r), per row, in fp64,
    with the biased variance; returns (y, mean, rstd).  gamma = None means 1,
    beta = None means 0; r (optional) is added to the normalised output."""
    x = np.asarray(x64, dtype=np.float64)
    n = x.shape[-1]
    if n == 0:
        raise ValueError("LayerNorm needs a non-empty row")
    mean = x.sum(axis=-1) / n
    centred = x - mean[..., None]
    var = (centred * centred).sum(axis=-1) / n
    rstd = 1.0 / np.sqrt(var + float(eps))
    y = centred * rstd[..., None]
    if gamma64 is not None:
        y = y * np.asarray(gamma64, dtype=np.float64).reshape(-1)[None, :]
    if beta64 is not None:
        y = y + np.asarray(beta64, dtype=np.float64).reshape(-1)[None, :]
    if r64 is not None:
        y = y + np.asarray(r64, dtype=np.float64)
    return y, mean, rstd


def layer_norm_reference(x_bits, dtype, gamma_bits=None, beta_bits=None, eps: float = LN_EPS, residual_bits=None):
    """LayerNorm of 16-bit inputs (bit patterns), every parameter widened exactly."""
    return layer_norm(widen(x_bits, dtype), None if gamma_bits is None else widen(gamma_bits, dtype),
                      None if beta_bits is None else widen(beta_bits, dtype), eps,
                      None if residual_bits is None else widen(residual_bits, dtype))
