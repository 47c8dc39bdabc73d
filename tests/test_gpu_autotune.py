"""Autotuning through the plan options ([bias-fusion] page, body, checklist:
autotuning is requested through plan()'s options) on the GPU: the first
execute of an autotune plan times every tile config that fits and keeps the
fastest.  Each case checks that first execute's outputs against the CPU
oracle, that the plan left the pending state for a valid config id, and that
a second execute (now of the chosen config only) reproduces the first bit for
bit.  A capturing stream refuses a pending autotune and leaves it pending."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import bias_tensor, compare, compare_bias_grad, fp8_to_device, scale_tensor, to_device, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def _pending(mm):
    return "autotune=pending" in mm.describe()


def _tuned(mm, first_cfg):
    import dense_gemm_epilogue_fp16_amd as egm
    assert not _pending(mm), mm.describe()
    cfg = egm.egm_plan_config(mm._plan)
    assert 0 <= cfg < egm.egm_num_configs(), cfg
    print(f"  default config {first_cfg} -> tuned config {cfg}: {mm.describe()}", flush=True)
    return cfg


# (m, n, k, dtype, epilog, bias layout, fused): ragged shapes for every tile,
# and the bias-fusion page's worked example shape (1024 x 512 x 2048, bias (m,1))
CASES = [
    (300, 264, 136, "fp16", "RELU_AUX_BIAS", "row", True),
    (300, 264, 136, "bf16", "GELU_BIAS", "col", True),
    (1024, 512, 2048, "fp16", "RELU_BIAS", "row", True),
    (1024, 512, 2048, "fp16", "BIAS", "row", False),
    (520, 392, 328, "bf16", "BIAS_RESIDUAL", "col", False),
]


@pytest.mark.parametrize("m,n,k,dtype,epilog,layout,fused", CASES)
def test_autotune_forward(m, n, k, dtype, epilog, layout, fused):
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    print(f"[autotune {m}x{n}x{k} {dtype} {epilog} {layout} fused={fused}]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=71, a_std=1.0, b_std=1.0 / np.sqrt(k) / 2, bias_layout=layout,
                          bias_std=0.5, residual_std=0.5 if epilog == "BIAS_RESIDUAL" else None)
    ins = {"bias": bias_tensor(ops.bias, layout, dtype)}
    if epilog == "BIAS_RESIDUAL":
        ins["residual"] = to_device(ops.residual, dtype)
    with egm.Matmul(to_device(ops.a, dtype), to_device(ops.b, dtype)) as mm:
        mm.plan(epilog, ins, fused=fused, autotune=True)
        assert _pending(mm)
        first_cfg = egm.egm_plan_config(mm._plan)
        out1 = mm.execute()
        torch.cuda.synchronize()
        _tuned(mm, first_cfg)
        out2 = mm.execute()
        torch.cuda.synchronize()
    d1, m1 = (out1 if isinstance(out1, tuple) else (out1, None))
    d2, m2 = (out2 if isinstance(out2, tuple) else (out2, None))
    y, z, mref = eo.reference(ops.a, ops.b, dtype, epilog, ops.bias, layout,
                              ops.residual if epilog == "BIAS_RESIDUAL" else None)
    st = compare(to_host_bits(d1), y, dtype, z=z, mask=None if m1 is None else m1.cpu().numpy(), mask_ref=mref,
                 unfused=not fused)
    print(f"  {st}", flush=True)
    assert np.array_equal(to_host_bits(d1), to_host_bits(d2))
    if m1 is not None:
        assert torch.equal(m1, m2)


@pytest.mark.parametrize("layout,fused", [("col", True), ("row", True), ("col", False)])
def test_autotune_bias_gradient(layout, fused):
    """DRELU_BGRAD: the workspace covers every config autotuning may launch."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype = 1000, 520, 264, "bf16"
    print(f"[autotune DRELU_BGRAD {m}x{n}x{k} {layout} fused={fused}]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=72, a_std=1.0, b_std=1.0 / np.sqrt(k), bias_layout=layout)
    mask = np.random.default_rng(73).integers(0, 256, size=(m, n // 8), dtype=np.uint8)
    shape = (m, 1) if layout == "row" else (1, n)
    grad = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    aux = torch.from_numpy(mask).cuda()
    with egm.Matmul(to_device(ops.a, dtype), to_device(ops.b, dtype)) as mm:
        mm.plan("DRELU_BGRAD", {"bias_grad": grad}, fused=fused, autotune=True)
        assert _pending(mm)
        first_cfg = egm.egm_plan_config(mm._plan)
        d1, g1 = mm.execute(aux=aux)
        torch.cuda.synchronize()
        g1 = g1.clone()
        _tuned(mm, first_cfg)
        d2, g2 = mm.execute(aux=aux)
        torch.cuda.synchronize()
    dz, g_ref, bound = eo.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, layout)
    st = compare(to_host_bits(d1), dz, dtype, unfused=not fused)
    gs = compare_bias_grad(g1.double().cpu().numpy().reshape(-1), g_ref, bound, d_ref=None if fused else dz,
                           dtype=dtype, layout=layout)
    print(f"  D {st} grad {gs}", flush=True)
    assert np.array_equal(to_host_bits(d1), to_host_bits(d2))
    assert torch.equal(g1, g2)


def test_autotune_fp8():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k = 520, 400, 272
    print(f"[autotune fp8 e4m3xe5m2 {m}x{n}x{k} RELU_AUX_BIAS]", flush=True)
    f8 = W.fp8_operands(m, n, k, "e4m3", "e5m2", "fp16", seed=74, bias_layout="col")
    with egm.Matmul(fp8_to_device(f8.a, "e4m3"), fp8_to_device(f8.b, "e5m2"), scale_a=scale_tensor(f8.scale_a),
                    scale_b=scale_tensor(f8.scale_b), out_dtype=torch.float16) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": bias_tensor(f8.bias, "col", "fp16")}, autotune=True)
        first_cfg = egm.egm_plan_config(mm._plan)
        d1, m1 = mm.execute()
        torch.cuda.synchronize()
        _tuned(mm, first_cfg)
        d2, m2 = mm.execute()
        torch.cuda.synchronize()
    y, z, mref = eo.reference_fp8(f8.a, f8.b, "e4m3", "e5m2", f8.scale_a, f8.scale_b, "fp16", "RELU_AUX_BIAS",
                                  f8.bias, "col")
    print(" ", compare(to_host_bits(d1), y, "fp16", z=z, mask=m1.cpu().numpy(), mask_ref=mref), flush=True)
    assert np.array_equal(to_host_bits(d1), to_host_bits(d2)) and torch.equal(m1, m2)


def test_autotune_refused_while_capturing():
    """The first execute of an autotune plan waits on the host for its
    timings, which a graph cannot record: under capture it returns
    EGM_ERR_NOT_SUPPORTED, enqueues nothing and leaves the plan pending; run
    eagerly afterwards it tunes and matches a plain plan's config choice set."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype = 256, 256, 512, "fp16"
    print(f"[autotune under capture {m}x{n}x{k}]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=75, bias_layout="row")
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    bias = bias_tensor(ops.bias, "row", dtype)
    d = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    x = torch.zeros(16, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("BIAS", {"bias": bias}, autotune=True)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        statuses = []
        with torch.cuda.graph(g, stream=side):
            x.add_(1.0)  # the graph must not be empty
            raw = torch.cuda.current_stream().cuda_stream
            statuses.append(egm.egm_execute(mm._plan, a.data_ptr(), b.data_ptr(), d.data_ptr(), stream=raw,
                                            raw_status=True))
        torch.cuda.synchronize()
        assert statuses == [egm.EGM_ERR_NOT_SUPPORTED], statuses
        assert _pending(mm)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isnan(d).all()  # nothing of the GEMM was recorded
        assert float(x[0]) == 1.0
        out = mm.execute(out=d)
        torch.cuda.synchronize()
        assert not _pending(mm)
    y, _, _ = eo.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, "row")
    print(" ", compare(to_host_bits(out), y, dtype), flush=True)
