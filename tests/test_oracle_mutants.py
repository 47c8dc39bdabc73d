"""Plant one plausible mistake at a time in the CPU oracle and check that at
least one pin fails for it (CPU only; the oracle is restored after each case)."""
import numpy as np
import pytest

from oracle import egm_oracle as eo
from oracle_pins import PINS

_orig = {name: getattr(eo, name) for name in dir(eo) if not name.startswith("__")}


def _drop_bias(p, bias64, layout):
    return p


def _swapped_layout(p, bias64, layout):
    return _orig["add_bias"](p, bias64, "col" if layout == "row" else "row")


def _drop_last_k(a64, b64):
    if a64.shape[1] <= 1:
        return _orig["product"](a64, b64)
    return a64[:, :-1] @ b64[:-1]


def _reversed_k(a64, b64):
    return a64 @ b64[::-1]


def _gelu_minus(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 - np.tanh(eo.GELU_C0 * (z + eo.GELU_C1 * z ** 3)))


def _gelu_sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-1.702 * z))


def _mask_msb(z):
    return np.packbits(np.asarray(z) > 0.0, axis=1, bitorder="big")


def _mask_ge(z):
    return np.packbits(np.asarray(z) >= 0.0, axis=1, bitorder="little")


def _relu_abs(z):
    return np.abs(np.asarray(z, dtype=np.float64))


def _epilog_residual_minus(z, epilog, r64=None):
    if epilog == "BIAS_RESIDUAL":
        return np.asarray(z) - np.asarray(r64)
    return _orig["apply_epilog"](z, epilog, r64)


def _epilog_gelu_on_bias_only(z, epilog, r64=None):
    if epilog == "GELU_BIAS":
        return _orig["relu"](z)
    return _orig["apply_epilog"](z, epilog, r64)


def _round_trunc(y, dtype):
    y = np.asarray(y, dtype=np.float64)
    if dtype == "fp16":
        sig, emin = 11, -14
    else:
        sig, emin = 8, -126
    _, e = np.frexp(y)
    q = np.ldexp(np.ones_like(y), np.maximum(e - 1, emin) - (sig - 1))
    r = np.trunc(y / q) * q
    if dtype == "fp16":
        return r.astype(np.float16).view(np.uint16)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _round_via_f32(y, dtype):
    # double rounding: fp64 -> fp32 -> 16 bit
    return _orig["round_to_bits"](np.asarray(y, np.float64).astype(np.float32).astype(np.float64), dtype)


def _widen_bf16_shift15(bits, dtype):
    if dtype == "bf16":
        return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _orig["widen"](bits, dtype)


def _unpack_msb(mask, n):
    return np.unpackbits(np.asarray(mask, dtype=np.uint8), axis=1, bitorder="big").astype(bool)


def _drelu_inverted(p, mask):
    p = np.asarray(p, dtype=np.float64)
    return np.where(_orig["unpack_mask"](mask, p.shape[1]), 0.0, p)


def _bias_grad_wrong_axis(dz, layout):
    return _orig["bias_grad"](dz, "row" if layout == "col" else "col")


def _bias_grad_mean(dz, layout):
    dz = np.asarray(dz, dtype=np.float64)
    return dz.mean(axis=0) if layout == "col" else dz.mean(axis=1)


def _bound_without_k(a64, b64, mask, layout):
    full = _orig["bias_grad_error_bound"](a64, b64, mask, layout)
    k = np.asarray(a64).shape[1]
    n_red = np.asarray(a64).shape[0] if layout == "col" else np.asarray(b64).shape[1]
    return full * n_red / (k + n_red)


def _fp8_subnormal_as_normal(bits, fmt):
    ebits, mbits, bias = eo.FP8_FORMATS[fmt]
    v = _orig["decode_fp8"](bits, fmt)
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e, m = (b >> mbits) & ((1 << ebits) - 1), b & ((1 << mbits) - 1)
    implicit = np.ldexp((m + (1 << mbits)).astype(np.float64), -bias - mbits)
    return np.where(e == 0, np.where(b >> 7 == 1, -implicit, implicit), v)


def _fp8_e5m2_no_infinity(bits, fmt):
    v = _orig["decode_fp8"](bits, fmt)
    if fmt != "e5m2":
        return v
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e, m = (b >> 2) & 31, b & 3
    big = np.ldexp((m + 4).astype(np.float64), 31 - 15 - 2)
    return np.where(e == 31, np.where(b >> 7 == 1, -big, big), v)


def _fp8_scale_ignored(a, b, fa, fb, sa, sb, *args, **kw):
    return _orig["reference_fp8"](a, b, fa, fb, np.float32(1), np.float32(1), *args, **kw)


def _fp8_only_scale_a(a, b, fa, fb, sa, sb, *args, **kw):
    return _orig["reference_fp8"](a, b, fa, fb, sa, np.float32(1), *args, **kw)


def _fp8_scale_on_bias(a, b, fa, fb, sa, sb, out, epilog, bias_bits=None, bias_layout=None,
                       residual_bits=None, rows=None):
    s = float(np.float32(sa)) * float(np.float32(sb))
    z = eo.product(eo.decode_fp8(a, fa), eo.decode_fp8(b, fb))
    if epilog != "DEFAULT":
        z = eo.add_bias(z, eo.widen(bias_bits, out), bias_layout)
    z = z * s
    r64 = eo.widen(residual_bits, out) if residual_bits is not None else None
    y = eo.apply_epilog(z, epilog, r64)
    return y, z, (eo.relu_mask(z) if epilog == "RELU_AUX_BIAS" else None)


def _ln_unbiased(x64, gamma64=None, beta64=None, eps=1e-5, r64=None):
    x = np.asarray(x64, dtype=np.float64)
    n = x.shape[-1]
    y, mean, _ = _orig["layer_norm"](x, None, None, 0.0)
    var = ((x - mean[..., None]) ** 2).sum(axis=-1) / max(n - 1, 1)
    rstd = 1 / np.sqrt(var + eps)
    y = (x - mean[..., None]) * rstd[..., None]
    y = y * (1 if gamma64 is None else np.asarray(gamma64)[None, :]) + (0 if beta64 is None else np.asarray(beta64)[None, :])
    return (y if r64 is None else y + r64), mean, rstd


def _ln_eps_outside(x64, gamma64=None, beta64=None, eps=1e-5, r64=None):
    x = np.asarray(x64, dtype=np.float64)
    mean = x.mean(axis=-1)
    rstd = 1 / (np.sqrt(((x - mean[..., None]) ** 2).mean(axis=-1)) + eps)
    y = (x - mean[..., None]) * rstd[..., None]
    y = y * (1 if gamma64 is None else np.asarray(gamma64)[None, :]) + (0 if beta64 is None else np.asarray(beta64)[None, :])
    return (y if r64 is None else y + r64), mean, rstd


def _ln_residual_before(x64, gamma64=None, beta64=None, eps=1e-5, r64=None):
    x = np.asarray(x64, dtype=np.float64) + (0 if r64 is None else np.asarray(r64))
    return _orig["layer_norm"](x, gamma64, beta64, eps, None)


def _ln_gamma_beta_swapped(x64, gamma64=None, beta64=None, eps=1e-5, r64=None):
    return _orig["layer_norm"](x64, beta64, gamma64, eps, r64)


def _ln_column_stats(x64, gamma64=None, beta64=None, eps=1e-5, r64=None):
    y, mean, rstd = _orig["layer_norm"](np.asarray(x64, dtype=np.float64).T, None, None, eps, None)
    y = y.T * (1 if gamma64 is None else np.asarray(gamma64)[None, :]) + (0 if beta64 is None else np.asarray(beta64)[None, :])
    return (y if r64 is None else y + r64), mean, rstd


def _ulp_doubled(y, dtype):
    return 2.0 * _orig["ulp"](y, dtype)


def _ulp_one_binade_low(y, dtype):
    return 0.5 * _orig["ulp"](y, dtype)


def _ln_ref_gamma_beta_swapped(x_bits, dtype, gamma_bits=None, beta_bits=None, eps=1e-5, residual_bits=None):
    return _orig["layer_norm_reference"](x_bits, dtype, beta_bits, gamma_bits, eps, residual_bits)


def _ln_ref_residual_dropped(x_bits, dtype, gamma_bits=None, beta_bits=None, eps=1e-5, residual_bits=None):
    return _orig["layer_norm_reference"](x_bits, dtype, gamma_bits, beta_bits, eps, None)


def _ln_ref_default_eps(x_bits, dtype, gamma_bits=None, beta_bits=None, eps=1e-5, residual_bits=None):
    return _orig["layer_norm_reference"](x_bits, dtype, gamma_bits, beta_bits, 1e-5, residual_bits)


def _reference_rows_unsliced_bias(a_bits, b_bits, dtype, epilog, bias_bits=None, bias_layout=None,
                                  residual_bits=None, rows=None):
    # a sampled-row reference that forgets to slice a per-row bias: it uses the
    # first len(rows) bias values instead of the sampled rows' own
    if rows is not None and bias_layout == "row" and bias_bits is not None:
        rows = np.asarray(rows)
        y, z, m = _orig["reference"](np.asarray(a_bits)[rows], b_bits, dtype, epilog,
                                     np.asarray(bias_bits).reshape(-1)[: len(rows)], bias_layout,
                                     None if residual_bits is None else np.asarray(residual_bits)[rows])
        return y, z, m
    return _orig["reference"](a_bits, b_bits, dtype, epilog, bias_bits, bias_layout, residual_bits, rows)


def _reference_mask_after_relu(a_bits, b_bits, dtype, epilog, bias_bits=None, bias_layout=None,
                               residual_bits=None, rows=None):
    # the mask taken from the activated output with >= (every bit set)
    y, z, m = _orig["reference"](a_bits, b_bits, dtype, epilog, bias_bits, bias_layout, residual_bits, rows)
    if m is not None:
        m = np.packbits(y >= 0.0, axis=1, bitorder="little")
    return y, z, m


def _backward_reference_no_mask(a_bits, b_bits, dtype, epilog, mask, bias_layout=None):
    full = np.full_like(np.asarray(mask, dtype=np.uint8), 0xFF)
    return _orig["backward_reference"](a_bits, b_bits, dtype, epilog, full, bias_layout)


def _backward_reference_axis_swapped(a_bits, b_bits, dtype, epilog, mask, bias_layout=None):
    swapped = None if bias_layout is None else ("row" if bias_layout == "col" else "col")
    return _orig["backward_reference"](a_bits, b_bits, dtype, epilog, mask, swapped)


MUTANTS = {
    "reference_rows_unsliced_bias": ("reference", _reference_rows_unsliced_bias),
    "reference_mask_after_relu": ("reference", _reference_mask_after_relu),
    "backward_reference_no_mask": ("backward_reference", _backward_reference_no_mask),
    "backward_reference_axis_swapped": ("backward_reference", _backward_reference_axis_swapped),
    "ulp_doubled": ("ulp", _ulp_doubled),
    "ulp_halved": ("ulp", _ulp_one_binade_low),
    "ln_ref_gamma_beta_swapped": ("layer_norm_reference", _ln_ref_gamma_beta_swapped),
    "ln_ref_residual_dropped": ("layer_norm_reference", _ln_ref_residual_dropped),
    "ln_ref_eps_ignored": ("layer_norm_reference", _ln_ref_default_eps),
    "ln_unbiased_variance": ("layer_norm", _ln_unbiased),
    "ln_eps_outside_sqrt": ("layer_norm", _ln_eps_outside),
    "ln_residual_before_norm": ("layer_norm", _ln_residual_before),
    "ln_gamma_beta_swapped": ("layer_norm", _ln_gamma_beta_swapped),
    "ln_column_statistics": ("layer_norm", _ln_column_stats),
    "fp8_e4m3_bias_8": ("FP8_FORMATS", {"e4m3": (4, 3, 8), "e5m2": (5, 2, 15)}),
    "fp8_subnormal_as_normal": ("decode_fp8", _fp8_subnormal_as_normal),
    "fp8_e5m2_no_infinity": ("decode_fp8", _fp8_e5m2_no_infinity),
    "fp8_scale_ignored": ("reference_fp8", _fp8_scale_ignored),
    "fp8_only_scale_a": ("reference_fp8", _fp8_only_scale_a),
    "fp8_scale_on_bias": ("reference_fp8", _fp8_scale_on_bias),
    "bias_dropped": ("add_bias", _drop_bias),
    "bias_layout_swapped": ("add_bias", _swapped_layout),
    "product_drops_last_k": ("product", _drop_last_k),
    "product_reversed_k": ("product", _reversed_k),
    "gelu_sign": ("gelu_tanh", _gelu_minus),
    "gelu_sigmoid_form": ("gelu_tanh", _gelu_sigmoid),
    "gelu_constant": ("GELU_C1", 0.0447),
    "mask_msb_first": ("relu_mask", _mask_msb),
    "mask_ge_zero": ("relu_mask", _mask_ge),
    "relu_is_abs": ("relu", _relu_abs),
    "residual_subtracted": ("apply_epilog", _epilog_residual_minus),
    "gelu_epilog_wrong_activation": ("apply_epilog", _epilog_gelu_on_bias_only),
    "round_truncates": ("round_to_bits", _round_trunc),
    "round_twice_via_fp32": ("round_to_bits", _round_via_f32),
    "widen_bf16_wrong_shift": ("widen", _widen_bf16_shift15),
    "mask_unpacked_msb_first": ("unpack_mask", _unpack_msb),
    "drelu_mask_inverted": ("drelu", _drelu_inverted),
    "bias_grad_wrong_axis": ("bias_grad", _bias_grad_wrong_axis),
    "bias_grad_mean_not_sum": ("bias_grad", _bias_grad_mean),
    "bias_grad_bound_drops_k_term": ("bias_grad_error_bound", _bound_without_k),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(eo, attr, bad)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(eo)
            except Exception as exc:  # AssertionError or a shape error both count
                caught.append((pin.__name__, type(exc).__name__))
                break
    assert caught, f"no pin caught the planted mistake {name!r}"
