"""Harness glue for the GPU parity tests: moves seeded operands to the device,
runs the HIP path through the C ABI (via the thin binding) and compares the
result with the CPU oracle element by element."""
from __future__ import annotations

import numpy as np

from oracle import egm_oracle as eo

TOL = eo.TOLERANCE  # fp16 out: 1e-2, bf16 out: 2e-2
MASK_EXEMPT = 1e-2  # mask bits are judged only where |Z| > this


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == "fp16" else torch.bfloat16


def to_device(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bias_tensor(bits, layout, dtype):
    t = to_device(bits, dtype)
    return t.reshape(-1, 1) if layout == "row" else t.reshape(1, -1)


def run(ops, epilog, *, fused=True, force_config=-1, group_m=0, a=None, b=None, residual=None):
    """Run one epilog on Operands through the binding; returns (D bits, mask or None)."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = to_device(ops.a, ops.dtype) if a is None else a
    b = to_device(ops.b, ops.dtype) if b is None else b
    ins = {}
    if epilog != "DEFAULT":
        ins["bias"] = bias_tensor(ops.bias, ops.bias_layout, ops.dtype)
    if epilog == "BIAS_RESIDUAL":
        ins["residual"] = to_device(ops.residual, ops.dtype) if residual is None else residual
    with egm.Matmul(a, b) as mm:
        mm.plan(epilog=epilog, epilog_inputs=ins, fused=fused, force_config=force_config, group_m=group_m)
        out = mm.execute()
        torch.cuda.synchronize()
    if isinstance(out, tuple):
        return to_host_bits(out[0]), out[1].cpu().numpy()
    return to_host_bits(out), None


def compare(d_bits, y, dtype, *, z=None, mask=None, mask_ref=None, unfused=False, tol=None):
    """Assert D matches the unrounded oracle Y; returns statistics.

    Fused path: max |D - Y| <= tol.  Two-kernel path (the product is rounded
    to 16 bits before the epilogue, a second rounding): |D - Y| <= tol + ulp(Y)/2.
    Mask: bit-exact wherever |Z| > 1e-2.
    """
    tol = TOL[dtype] if tol is None else tol
    d = eo.widen(d_bits, dtype)
    assert d.shape == y.shape, (d.shape, y.shape)
    assert np.isfinite(d).all(), "non-finite output"
    err = np.abs(d - y)
    bound = tol + (0.5 * eo.ulp(y, dtype) if unfused else 0.0)
    bad = err > bound
    stats = {"max_abs_err": float(err.max()) if err.size else 0.0, "n_out": int(err.size),
             "n_over": int(bad.sum())}
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} of {err.size} outputs exceed the bound; first at {tuple(i)}: "
                             f"D={d[tuple(i)]!r} Y={y[tuple(i)]!r} |err|={err[tuple(i)]:.3g}")
    if mask_ref is not None:
        assert mask is not None and mask.shape == mask_ref.shape and mask.dtype == np.uint8
        got = np.unpackbits(mask, axis=1, bitorder="little")
        want = np.unpackbits(mask_ref, axis=1, bitorder="little")
        judged = np.abs(z) > MASK_EXEMPT
        mism = (got != want) & judged
        stats["mask_mismatch"] = int(mism.sum())
        stats["mask_exempt"] = int((~judged).sum())
        assert not mism.any(), f"{int(mism.sum())} mask bits differ where |Z| > {MASK_EXEMPT}"
    return stats


def exact_bits(y, dtype):
    """The single correct rounding of an exact oracle result (integer tests)."""
    return eo.round_to_bits(y, dtype)


def run_backward(ops, epilog, mask, layout=None, *, fused=True, force_config=-1):
    """Run DRELU / DRELU_BGRAD on Operands (A.B is the incoming gradient) with
    a host mask [m, n/8]; returns (D bits, bias gradient as float64 or None)."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a, b = to_device(ops.a, ops.dtype), to_device(ops.b, ops.dtype)
    aux = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    ins = {}
    if epilog == "DRELU_BGRAD":
        shape = (ops.m, 1) if layout == "row" else (1, ops.n)
        # poisoned: every value must be written by the library
        ins["bias_grad"] = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan(epilog=epilog, epilog_inputs=ins, fused=fused, force_config=force_config)
        out = mm.execute(aux=aux)
        torch.cuda.synchronize()
    if isinstance(out, tuple):
        return to_host_bits(out[0]), out[1].double().cpu().numpy().reshape(-1)
    return to_host_bits(out), None


def compare_bias_grad(got, want, bound, *, d_ref=None, dtype=None, layout=None):
    """The bias gradient against the oracle within its fp32 error bound; for
    the two-kernel path (sums of the rounded D) pass the oracle dZ so the
    rounding of each summed value (half an ulp) widens the bound."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), "non-finite bias gradient"
    b = bound.copy()
    if d_ref is not None:
        b = b + eo.bias_grad(0.5 * eo.ulp(d_ref, dtype) * (d_ref != 0), layout)
    err = np.abs(got - want)
    bad = err > b
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{int(bad.sum())} of {err.size} bias-gradient values exceed the bound; first at {i}: "
                             f"got={got[i]!r} want={want[i]!r} bound={b[i]:.3g}")
    return {"max_abs_err": float(err.max()) if err.size else 0.0}


def fp8_to_device(bits, fmt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).cuda()
    return t.view(torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2)


def scale_tensor(value):
    import torch
    return torch.tensor([float(np.float32(value))], dtype=torch.float32, device="cuda")


def run_fp8(ops, epilog, *, fused=True, force_config=-1, null_scales=False):
    """Run one epilog on Fp8Operands through the binding; returns (D bits, mask or None)."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a, b = fp8_to_device(ops.a, ops.a_fmt), fp8_to_device(ops.b, ops.b_fmt)
    sa = None if null_scales else scale_tensor(ops.scale_a)
    sb = None if null_scales else scale_tensor(ops.scale_b)
    ins = {}
    if epilog != "DEFAULT":
        ins["bias"] = bias_tensor(ops.bias, ops.bias_layout, ops.out_dtype)
    if epilog == "BIAS_RESIDUAL":
        ins["residual"] = to_device(ops.residual, ops.out_dtype)
    with egm.Matmul(a, b, scale_a=sa, scale_b=sb, out_dtype=torch_dtype(ops.out_dtype)) as mm:
        mm.plan(epilog=epilog, epilog_inputs=ins, fused=fused, force_config=force_config)
        out = mm.execute()
        torch.cuda.synchronize()
    if isinstance(out, tuple):
        return to_host_bits(out[0]), out[1].cpu().numpy()
    return to_host_bits(out), None
