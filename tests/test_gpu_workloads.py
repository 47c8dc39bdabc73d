"""The named workloads on the HIP path vs the CPU oracle (GPU).

Inputs are the seeded synthetic operands of ``egm_workloads`` at the full
sizes; the launch configuration is the per-shape default that bench.py times.
The largest workload is checked on 4096 sampled rows (first and last row
always included), every column.
"""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import compare, run, to_device, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_gemm(name, epilog, fused=True):
    ops = W.workload_operands(name)
    d, mask = run(ops, epilog, fused=fused)
    y, z, mref = eo.reference(ops.a, ops.b, ops.dtype, epilog, ops.bias, ops.bias_layout)
    st = compare(d, y, ops.dtype, z=z, mask=mask, mask_ref=mref, unfused=not fused)
    print(f"[{name} {epilog} {'fused' if fused else 'unfused'}] {st}", flush=True)
    return st


@pytest.mark.parametrize("fused", [True, False])
def test_small_square_bias(fused):
    _check_gemm("gemm_bias_fp16_256x256x512", "BIAS", fused)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("epilog", ["BIAS", "RELU_BIAS"])
def test_worked_example_shape(epilog, fused):
    _check_gemm("gemm_bias_relu_fp16_1024x512x2048", epilog, fused)


@pytest.mark.slow
def test_ffn_chain():
    """Up-projection GELU_BIAS then down-projection BIAS_RESIDUAL (R = X).
    (i) the up-projection against the oracle; (ii) the down-projection run on
    the oracle's own rounded H (uploaded), against the oracle on that H; (iii)
    the GPU chain (down-projection on the GPU's H) against the oracle's chain.
    No GPU output is ever an oracle input."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    f = W.ffn_operands()
    x, w1, w2 = to_device(f.x, "bf16"), to_device(f.w1, "bf16"), to_device(f.w2, "bf16")
    b1 = to_device(f.b1, "bf16").reshape(1, -1)
    b2 = to_device(f.b2, "bf16").reshape(1, -1)
    y_up, _, _ = eo.reference(f.x, f.w1, "bf16", "GELU_BIAS", f.b1, "col")
    h_ref = eo.round_to_bits(y_up, "bf16")
    with egm.Matmul(x, w1) as up, egm.Matmul(torch.empty((f.tokens, f.ffn), dtype=torch.bfloat16, device="cuda"),
                                             w2) as down:
        up.plan("GELU_BIAS", {"bias": b1})
        h = up.execute()
        down.plan("BIAS_RESIDUAL", {"bias": b2, "residual": x})
        d_chain = down.execute(a=h)
        d_on_ref_h = down.execute(a=to_device(h_ref, "bf16"))
        torch.cuda.synchronize()
    print("[ffn up]", compare(to_host_bits(h), y_up, "bf16"), flush=True)
    y_dn, _, _ = eo.reference(h_ref, f.w2, "bf16", "BIAS_RESIDUAL", f.b2, "col", f.x)
    print("[ffn down, oracle H]", compare(to_host_bits(d_on_ref_h), y_dn, "bf16"), flush=True)
    print("[ffn chain, GPU H]", compare(to_host_bits(d_chain), y_dn, "bf16"), flush=True)


@pytest.mark.slow
def test_square_relu_aux_bias():
    _check_gemm("gemm_relu_aux_bias_bf16_8192x8192x8192", "RELU_AUX_BIAS")


@pytest.mark.slow
@pytest.mark.parametrize("fused", [True, False])
def test_backward_workload(fused):
    """The 8192^3 DRELU_BGRAD workload at full size, in the launch
    configuration bench.py times: every output of D and the whole (1,n)
    gradient against the oracle."""
    from parity import compare_bias_grad, run_backward
    name = "drelu_bgrad_bf16_8192x8192x8192"
    ops, mask = W.backward_operands(name)
    d, grad = run_backward(ops, "DRELU_BGRAD", mask, ops.bias_layout, fused=fused)
    dz, g_ref, bound = eo.backward_reference(ops.a, ops.b, ops.dtype, "DRELU_BGRAD", mask, ops.bias_layout)
    st = compare(d, dz, ops.dtype, unfused=not fused)
    gs = compare_bias_grad(grad, g_ref, bound, d_ref=None if fused else dz, dtype=ops.dtype, layout=ops.bias_layout)
    print(f"[{name} fused={fused}] D {st} grad {gs}", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("fused", [True, False])
def test_fp8_workload(fused):
    """The E4M3 8192^3 RELU_AUX_BIAS workload at full size, in the launch
    configuration bench.py times: every output and every mask bit."""
    from parity import run_fp8
    name = "gemm_relu_aux_bias_fp8e4m3_8192x8192x8192"
    ops = W.fp8_workload_operands(name)
    d, mask = run_fp8(ops, "RELU_AUX_BIAS", fused=fused)
    y, z, mref = eo.reference_fp8(ops.a, ops.b, ops.a_fmt, ops.b_fmt, ops.scale_a, ops.scale_b, ops.out_dtype,
                                  "RELU_AUX_BIAS", ops.bias, ops.bias_layout)
    st = compare(d, y, ops.out_dtype, z=z, mask=mask, mask_ref=mref, unfused=not fused)
    print(f"[{name} fused={fused}] {st}", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("fused", [True, False])
def test_largest_sampled_rows(fused):
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    name = "gemm_relu_bias_fp16_65536x16384x16384"
    ops = W.workload_operands(name)
    rows = W.sample_rows(ops.m, 4096, seed=1)
    a, b = to_device(ops.a, "fp16"), to_device(ops.b, "fp16")
    bias = to_device(ops.bias, "fp16").reshape(-1, 1)
    with egm.Matmul(a, b) as mm:
        mm.plan("RELU_BIAS", {"bias": bias}, fused=fused)
        d = mm.execute()
        sel = d.index_select(0, torch.from_numpy(rows).cuda())
        torch.cuda.synchronize()
    del a, d
    y, _, _ = eo.reference(ops.a, ops.b, "fp16", "RELU_BIAS", ops.bias, "row", rows=rows)
    st = compare(to_host_bits(sel), y, "fp16", unfused=not fused)
    print(f"[{name} fused={fused} rows={len(rows)}] {st}", flush=True)


@pytest.mark.parametrize("name", [n for n in W.WORKLOAD_ORDER if not n.startswith("ffn_")][:3] +
                         ["ffn_up", "ffn_down"])
def test_supplementary_unit_scale(name):
    """A ~ N(0,1), B ~ N(0,1)/sqrt(K), zero bias: the GEMM term itself is O(1)
    and is held to the same tolerance (the workloads' own scaling makes it
    O(K^-1/2) next to an N(0,1) bias)."""
    shapes = {"ffn_up": (4096, 4096, 1024, "bf16"), "ffn_down": (4096, 1024, 4096, "bf16")}
    if name in shapes:
        m, n, k, dtype = shapes[name]
    else:
        w = W.WORKLOADS[name]
        m, n, k, dtype = w.m, w.n, w.k, w.dtype
    ops = W.gemm_operands(m, n, k, dtype, seed=21, a_std=1.0, bias_layout="col")
    ops.bias = np.zeros_like(ops.bias)
    d, _ = run(ops, "BIAS")
    y, _, _ = eo.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, "col")
    print(f"[unit-scale {name}]", compare(d, y, dtype), flush=True)


@pytest.mark.slow
def test_supplementary_unit_scale_largest():
    """The unit-scale check at the largest shape, 65536 x 16384 x 16384 fp16:
    A ~ N(0,1), B ~ N(0,1)/sqrt(K), zero (m,1) bias, so the product term
    itself is O(1) (with the workload's own scaling it is about 0.008, below
    the 1e-2 tolerance, next to an N(0,1) bias).  Every column of 4096 sampled
    rows, first and last row included, in the launch configuration bench.py
    times.  K = 16384 is the only shape with 256 k-slabs per tile."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype = 65536, 16384, 16384, "fp16"
    print(f"[unit-scale {m}x{n}x{k} {dtype} BIAS row, 4096 sampled rows]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=22, a_std=1.0, bias_layout="row")
    ops.bias = np.zeros_like(ops.bias)
    rows = W.sample_rows(m, 4096, seed=1)
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    bias = to_device(ops.bias, dtype).reshape(-1, 1)
    with egm.Matmul(a, b) as mm:
        mm.plan("BIAS", {"bias": bias})
        d = mm.execute()
        sel = d.index_select(0, torch.from_numpy(rows).cuda())
        torch.cuda.synchronize()
    del a, b, d
    y, _, _ = eo.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, "row", rows=rows)
    assert float(np.std(y)) > 0.5  # the product term is O(1) here
    print(f"  {compare(to_host_bits(sel), y, dtype)}", flush=True)
