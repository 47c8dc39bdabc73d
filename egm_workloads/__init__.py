"""Seeded synthetic operands for D = epilogue(A.B) in fp16 / bf16.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle.  It holds no step of the method itself: only random draws, the single
fp32 -> fp16/bf16 rounding that turns a draw into an operand, the table of
workloads and the row sample used to check the largest one.

Operands are returned as numpy ``uint16`` arrays holding the exact 16-bit bit
patterns (numpy has no bf16 type); callers reinterpret them as fp16 / bf16.

Draw recipe (one fixed rule for every workload):
  * every tensor of a workload gets its own index ``t`` (in the order the
    workload lists them) and is drawn in chunks of ``CHUNK`` elements (row-major
    order); chunk ``c`` of tensor ``t`` of a workload with seed ``s`` comes from
    ``numpy.random.Generator(PCG64(SeedSequence(s, spawn_key=(t, c))))``,
    ``standard_normal(dtype=float32)``;
  * the fp32 draw is multiplied by the tensor's standard deviation in fp32 and
    rounded once, to nearest-even, to the operand type.
Chunks are independent streams, so the result does not depend on how many
threads fill them.

Workloads (distribution parameters are standard deviations; the pages write the
up/down-projection weights and biases as N(0, v) and v is read as a variance):
  gemm_bias_fp16_256x256x512        A,B ~ N(0,1)/sqrt(K), bias (m,1) ~ N(0,1), BIAS
  gemm_bias_relu_fp16_1024x512x2048 same draws, bias (m,1); BIAS then RELU_BIAS
                                    (the bias-fusion page's own worked example:
                                    m,n,k = 1024,512,2048, fp16, bias (m,1))
  ffn_bf16_4096x1024x4096           X[4096,1024] ~ N(0,1), W1[1024,4096] std 1/32,
                                    b1 (1,4096) std sqrt(0.02), W2[4096,1024]
                                    std 1/64, b2 (1,1024) std sqrt(0.02);
                                    up = GELU_BIAS, down = BIAS_RESIDUAL (R = X)
  gemm_relu_aux_bias_bf16_8192x8192x8192  A,B ~ N(0,1)/sqrt(K), bias (1,n) ~ N(0,1)
  gemm_relu_bias_fp16_65536x16384x16384   A,B ~ N(0,1)/sqrt(K), bias (m,1) ~ N(0,1)

fp8 operands (OCP E4M3 / E5M2) are made the way an fp8 producer makes them:
the fp32 draw gets a per-tensor scale amax / (largest finite fp8 value), is
divided by it in fp32 and rounded once, to nearest-even, to fp8 (torch's
conversion); the bits and the fp32 scale are the operand.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F16 = "fp16"
BF16 = "bf16"
DTYPES = (F16, BF16)

#: elements per independently seeded chunk
CHUNK = 1 << 22

_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)))


# --------------------------------------------------------------------------
# fp32 -> 16-bit operand rounding (round to nearest, ties to even)
# --------------------------------------------------------------------------
def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to fp16 or bf16 (nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32)
        # keep the top 16 bits, adding half an ulp plus the tie-breaking lsb
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns to float32 (for harness-side use)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# chunked, thread-parallel normal draws
# --------------------------------------------------------------------------
def _chunk_generator(seed: int, tensor_index: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(int(seed), spawn_key=(int(tensor_index), int(chunk)))
    return np.random.Generator(np.random.PCG64(ss))


def normal_bits(shape, std: float, dtype: str, seed: int, tensor_index: int) -> np.ndarray:
    """Draw N(0, std^2) in fp32, scale in fp32, round once to ``dtype``.

    Returns a C-contiguous uint16 array of ``shape``.
    """
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(total, dtype=np.uint16)
    nchunks = (total + CHUNK - 1) // CHUNK
    s32 = np.float32(std)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        g = _chunk_generator(seed, tensor_index, c)
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= s32
        out[lo:hi] = f32_to_bits(v, dtype)

    if nchunks <= 1 or _THREADS == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normal_f32(shape, std: float, seed: int, tensor_index: int) -> np.ndarray:
    """The same draws as ``normal_bits``, kept in fp32 (scaled by std in fp32)."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(total, dtype=np.float32)
    nchunks = (total + CHUNK - 1) // CHUNK
    s32 = np.float32(std)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        v = _chunk_generator(seed, tensor_index, c).standard_normal(hi - lo, dtype=np.float32)
        v *= s32
        out[lo:hi] = v

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# fp8 operands
# --------------------------------------------------------------------------
E4M3 = "e4m3"
E5M2 = "e5m2"
FP8 = (E4M3, E5M2)
#: largest finite value of each fp8 format
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}


def f32_to_fp8_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float32 values once (nearest-even, torch's conversion) to fp8,
    saturating at the largest finite value; return uint8 bits."""
    import torch
    if fmt not in FP8_MAX:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX[fmt], FP8_MAX[fmt])
    t = torch.from_numpy(x).to(torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2)
    return t.view(torch.uint8).numpy().copy()


def fp8_quantize(x: np.ndarray, fmt: str):
    """Per-tensor scaling: scale = amax / FP8_MAX (fp32; 1 for an all-zero
    tensor), q = fp8(x / scale).  Returns (uint8 bits, float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = np.float32(amax / FP8_MAX[fmt]) if amax > 0 else np.float32(1.0)
    return f32_to_fp8_bits(x / scale, fmt), scale


def integer_bits(shape, lo: int, hi: int, dtype: str, seed: int, tensor_index: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as exact fp16/bf16 patterns (|v| <= 256)."""
    assert -256 <= lo <= hi <= 256
    g = _chunk_generator(seed, tensor_index, 0)
    v = g.integers(lo, hi + 1, size=tuple(shape)).astype(np.float32)
    return f32_to_bits(v, dtype)


# --------------------------------------------------------------------------
# generic operand sets (used by the parity tests at arbitrary shapes)
# --------------------------------------------------------------------------
@dataclass
class Operands:
    """Bit patterns of one GEMM + epilogue problem (row-major)."""

    m: int
    n: int
    k: int
    dtype: str
    a: np.ndarray            # [m, k] uint16
    b: np.ndarray            # [k, n] uint16
    bias: np.ndarray | None  # [m] (row layout) or [n] (col layout) uint16
    bias_layout: str | None  # "row" = shape (m,1), "col" = shape (1,n)
    residual: np.ndarray | None = None  # [m, n] uint16
    meta: dict = field(default_factory=dict)


def gemm_operands(m, n, k, dtype, seed=0, *, a_std=None, b_std=None,
                  bias_layout="row", bias_std=1.0, residual_std=None) -> Operands:
    """Normal operands.  ``a_std``/``b_std`` default to 1/sqrt(K) (at least 1 row)."""
    kk = max(int(k), 1)
    a_std = 1.0 / math.sqrt(kk) if a_std is None else a_std
    b_std = 1.0 / math.sqrt(kk) if b_std is None else b_std
    a = normal_bits((m, k), a_std, dtype, seed, 0)
    b = normal_bits((k, n), b_std, dtype, seed, 1)
    bias = None
    if bias_layout is not None:
        blen = m if bias_layout == "row" else n
        bias = normal_bits((blen,), bias_std, dtype, seed, 2)
    r = None
    if residual_std is not None:
        r = normal_bits((m, n), residual_std, dtype, seed, 3)
    return Operands(m, n, k, dtype, a, b, bias, bias_layout, r)


def integer_operands(m, n, k, dtype, seed=0, *, lo=-2, hi=2, bias_layout="row",
                     bias_lo=-4, bias_hi=4, residual=False) -> Operands:
    """Small-integer operands: with K*hi*hi <= 256 every product, sum, bias and
    residual add is exact in fp32 and representable in fp16 and bf16."""
    a = integer_bits((m, k), lo, hi, dtype, seed, 0)
    b = integer_bits((k, n), lo, hi, dtype, seed, 1)
    bias = None
    if bias_layout is not None:
        blen = m if bias_layout == "row" else n
        bias = integer_bits((blen,), bias_lo, bias_hi, dtype, seed, 2)
    r = integer_bits((m, n), -4, 4, dtype, seed, 3) if residual else None
    return Operands(m, n, k, dtype, a, b, bias, bias_layout, r)


@dataclass
class Fp8Operands:
    """Bit patterns of one fp8 GEMM + epilogue problem (row-major)."""

    m: int
    n: int
    k: int
    a_fmt: str
    b_fmt: str
    out_dtype: str            # fp16 / bf16: the bias, residual and output type
    a: np.ndarray             # [m, k] uint8
    b: np.ndarray             # [k, n] uint8
    scale_a: np.float32
    scale_b: np.float32
    bias: np.ndarray | None   # [m] or [n] uint16 (out_dtype)
    bias_layout: str | None
    residual: np.ndarray | None = None  # [m, n] uint16 (out_dtype)
    meta: dict = field(default_factory=dict)


def fp8_operands(m, n, k, a_fmt, b_fmt, out_dtype, seed=0, *, a_std=1.0, b_std=None,
                 bias_layout="col", bias_std=1.0, residual_std=None) -> Fp8Operands:
    """Normal draws quantised per tensor (A ~ N(0, a_std^2), B ~ N(0, b_std^2),
    b_std = 1/sqrt(K) by default, so A.B is O(1)); bias and residual in out_dtype."""
    b_std = 1.0 / math.sqrt(max(int(k), 1)) if b_std is None else b_std
    a, sa = fp8_quantize(normal_f32((m, k), a_std, seed, 0), a_fmt)
    b, sb = fp8_quantize(normal_f32((k, n), b_std, seed, 1), b_fmt)
    bias = None
    if bias_layout is not None:
        bias = normal_bits((m if bias_layout == "row" else n,), bias_std, out_dtype, seed, 2)
    r = normal_bits((m, n), residual_std, out_dtype, seed, 3) if residual_std is not None else None
    return Fp8Operands(m, n, k, a_fmt, b_fmt, out_dtype, a, b, sa, sb, bias, bias_layout, r)


def fp8_integer_operands(m, n, k, a_fmt, b_fmt, out_dtype, seed=0, *, lo=-2, hi=2, bias_layout="col",
                         scale_a=1.0, scale_b=1.0, residual=False) -> Fp8Operands:
    """Small integers (exact in both fp8 formats) with power-of-two scales:
    every product, sum, scaling and bias add is exact in fp32."""
    g = _chunk_generator(seed, 0, 0)
    a = f32_to_fp8_bits(g.integers(lo, hi + 1, size=(m, k)).astype(np.float32), a_fmt)
    b = f32_to_fp8_bits(_chunk_generator(seed, 1, 0).integers(lo, hi + 1, size=(k, n)).astype(np.float32), b_fmt)
    bias = None
    if bias_layout is not None:
        bias = integer_bits((m if bias_layout == "row" else n,), -4, 4, out_dtype, seed, 2)
    r = integer_bits((m, n), -4, 4, out_dtype, seed, 3) if residual else None
    return Fp8Operands(m, n, k, a_fmt, b_fmt, out_dtype, a, b, np.float32(scale_a), np.float32(scale_b), bias,
                       bias_layout, r)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    k: int
    dtype: str
    epilogs: tuple
    bias_layout: str
    note: str = ""


WORKLOADS = {
    "gemm_bias_fp16_256x256x512": Workload(
        "gemm_bias_fp16_256x256x512", 256, 256, 512, F16, ("BIAS",), "row",
        "small case; oracle finishes in well under a second"),
    "gemm_bias_relu_fp16_1024x512x2048": Workload(
        "gemm_bias_relu_fp16_1024x512x2048", 1024, 512, 2048, F16, ("BIAS", "RELU_BIAS"), "row",
        "bias-fusion page's worked example shape; both epilogues on one input set"),
    "ffn_bf16_4096x1024x4096": Workload(
        "ffn_bf16_4096x1024x4096", 4096, 4096, 1024, BF16, ("GELU_BIAS", "BIAS_RESIDUAL"), "col",
        "transformer FFN: up 4096x4096x1024 GELU_BIAS, down 4096x1024x4096 BIAS_RESIDUAL(R=X)"),
    "gemm_relu_aux_bias_bf16_8192x8192x8192": Workload(
        "gemm_relu_aux_bias_bf16_8192x8192x8192", 8192, 8192, 8192, BF16, ("RELU_AUX_BIAS",), "col",
        "square; D plus packed 1-bit ReLU mask [8192, 1024] uint8"),
    "gemm_relu_bias_fp16_65536x16384x16384": Workload(
        "gemm_relu_bias_fp16_65536x16384x16384", 65536, 16384, 16384, F16, ("RELU_BIAS",), "row",
        "largest; the oracle checks 4096 sampled rows"),
}

#: workload names in table order (small -> large)
WORKLOAD_ORDER = tuple(WORKLOADS)

#: the backward of the square workload: the gradient reaching its ReLU output
#: (A.B with A ~ N(0,1), B ~ N(0,1)/sqrt(K)) through its mask, with the
#: gradient of its (1,n) bias.  The mask is drawn (uniform bytes, each bit 1
#: with probability 1/2, as for a ReLU over a zero-mean pre-activation) rather
#: than taken from a forward run, so that every oracle input is a draw.
BACKWARD_WORKLOADS = {
    "drelu_bgrad_bf16_8192x8192x8192": Workload(
        "drelu_bgrad_bf16_8192x8192x8192", 8192, 8192, 8192, BF16, ("DRELU_BGRAD",), "col",
        "backward of the square workload; bias gradient of its (1,n) bias"),
}


#: fp8 operands on the square workload, with its draws: A, B ~ N(0,1)/sqrt(K),
#: each quantised per tensor to E4M3 (the scale absorbs the 1/sqrt(K)), bias
#: (1,n) ~ N(0,1) and output in bf16
FP8_WORKLOADS = {
    "gemm_relu_aux_bias_fp8e4m3_8192x8192x8192": Workload(
        "gemm_relu_aux_bias_fp8e4m3_8192x8192x8192", 8192, 8192, 8192, BF16, ("RELU_AUX_BIAS",), "col",
        "square, E4M3 x E4M3 with per-tensor scales; bf16 bias and output, packed ReLU mask"),
}


def fp8_workload_operands(name: str, seed: int = 0) -> Fp8Operands:
    w = FP8_WORKLOADS[name]
    return fp8_operands(w.m, w.n, w.k, E4M3, E4M3, w.dtype, seed, a_std=1.0 / math.sqrt(w.k),
                        b_std=1.0 / math.sqrt(w.k), bias_layout=w.bias_layout)


@dataclass
class LayerNormOperands:
    """Bit patterns of one LayerNorm problem over rows of length n."""

    m: int
    n: int
    dtype: str
    x: np.ndarray                    # [m, n] uint16
    gamma: np.ndarray                # [n] uint16
    beta: np.ndarray                 # [n] uint16
    residual: np.ndarray | None = None  # [m, n] uint16


def layernorm_operands(m, n, dtype, seed=0, *, x_std=1.0, x_mean=0.5, gamma_std=0.05, beta_std=0.1,
                       residual_std=None) -> LayerNormOperands:
    """x ~ N(x_mean, x_std^2) (tensor 0), gamma ~ 1 + N(0, gamma_std^2) (1),
    beta ~ N(0, beta_std^2) (2), optional residual (3); each rounded once."""
    x = normal_f32((m, n), x_std, seed, 0) + np.float32(x_mean)
    g = normal_f32((n,), gamma_std, seed, 1) + np.float32(1.0)
    return LayerNormOperands(m, n, dtype, f32_to_bits(x, dtype), f32_to_bits(g, dtype),
                             normal_bits((n,), beta_std, dtype, seed, 2),
                             normal_bits((m, n), residual_std, dtype, seed, 3) if residual_std is not None else None)


#: LayerNorm after the FFN down-projection (its 4096 x 1024 hidden state), and
#: a large problem of the same row kernel for the HBM roofline
LAYERNORM_WORKLOADS = {
    "layernorm_bf16_4096x1024": Workload("layernorm_bf16_4096x1024", 4096, 1024, 0, BF16, ("LAYERNORM",), "col",
                                         "the FFN block's normalisation of its 4096 x 1024 output"),
    "layernorm_bf16_65536x16384": Workload("layernorm_bf16_65536x16384", 65536, 16384, 0, BF16, ("LAYERNORM",),
                                           "col", "2 GiB in, 2 GiB out: the row kernel at HBM scale"),
}


def mask_bits(m: int, n: int, seed: int, tensor_index: int) -> np.ndarray:
    """A packed [m, n/8] uint8 mask of independent fair bits."""
    if n % 8:
        raise ValueError("n must be a multiple of 8")
    return _uniform_bytes((m, n // 8), seed, tensor_index)


def _uniform_bytes(shape, seed: int, tensor_index: int) -> np.ndarray:
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint8)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        out[lo:hi] = _chunk_generator(seed, tensor_index, c).integers(0, 256, size=hi - lo, dtype=np.uint8)

    nchunks = (total + CHUNK - 1) // CHUNK
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def backward_operands(name: str, seed: int = 0):
    """(Operands of the gradient GEMM, packed mask) of a backward workload;
    tensor indices 0, 1 for A, B and 2 for the mask."""
    w = BACKWARD_WORKLOADS[name]
    a = normal_bits((w.m, w.k), 1.0, w.dtype, seed, 0)
    b = normal_bits((w.k, w.n), 1.0 / math.sqrt(w.k), w.dtype, seed, 1)
    ops = Operands(w.m, w.n, w.k, w.dtype, a, b, None, w.bias_layout)
    return ops, mask_bits(w.m, w.n, seed, 2)


def workload_operands(name: str, seed: int = 0) -> Operands:
    """Operands of a plain GEMM workload (all but the FFN chain)."""
    w = WORKLOADS[name]
    if name.startswith("ffn_"):
        raise ValueError("use ffn_operands() for the FFN chain")
    return gemm_operands(w.m, w.n, w.k, w.dtype, seed, bias_layout=w.bias_layout, bias_std=1.0)


@dataclass
class FFNOperands:
    tokens: int
    hidden: int
    ffn: int
    dtype: str
    x: np.ndarray   # [tokens, hidden]
    w1: np.ndarray  # [hidden, ffn]
    b1: np.ndarray  # [ffn]    (1, n) layout
    w2: np.ndarray  # [ffn, hidden]
    b2: np.ndarray  # [hidden] (1, n) layout


def ffn_operands(tokens=4096, hidden=1024, ffn=4096, dtype=BF16, seed=0) -> FFNOperands:
    """Transformer FFN pair; draw order X, W1, b1, W2, b2 (tensor indices 0..4)."""
    x = normal_bits((tokens, hidden), 1.0, dtype, seed, 0)
    w1 = normal_bits((hidden, ffn), 1.0 / math.sqrt(hidden), dtype, seed, 1)
    b1 = normal_bits((ffn,), math.sqrt(0.02), dtype, seed, 2)
    w2 = normal_bits((ffn, hidden), 1.0 / math.sqrt(ffn), dtype, seed, 3)
    b2 = normal_bits((hidden,), math.sqrt(0.02), dtype, seed, 4)
    return FFNOperands(tokens, hidden, ffn, dtype, x, w1, b1, w2, b2)


def sample_rows(m: int, count: int, seed: int = 1) -> np.ndarray:
    """Sorted, distinct row indices: first and last row always, the rest drawn
    without replacement from the interior with ``default_rng(seed)``."""
    if count >= m:
        return np.arange(m, dtype=np.int64)
    if count < 2:
        raise ValueError("need at least two rows")
    g = np.random.default_rng(seed)
    inner = g.choice(np.arange(1, m - 1, dtype=np.int64), count - 2, replace=False)
    return np.sort(np.concatenate([[0, m - 1], inner]).astype(np.int64))
