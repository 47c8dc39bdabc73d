"""Backward epilogues on the GPU against the CPU oracle, through the C ABI:
DRELU (the forward ReLU mask applied to the incoming gradient A.B) and
DRELU_BGRAD (plus the bias gradient).  The masks given to the oracle come from
the seeded generator or from the oracle's own forward pass."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import compare, compare_bias_grad, exact_bits, run, run_backward, to_host_bits

pytestmark = pytest.mark.gpu

CONFIGS = tuple(range(8))  # every tile config (5, 6, 7: 16x16x32 MFMA blocks)
RAGGED = (300, 264, 136)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def random_mask(m, n, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(m, n // 8), dtype=np.uint8)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_integer_exact(dtype, cfg, fused):
    """Integer gradients: D and both bias gradients exact, bit for bit."""
    m, n, k = RAGGED
    ops = W.integer_operands(m, n, k, dtype, seed=cfg + 40)
    mask = random_mask(m, n, cfg)
    dz, _, _ = eo.backward_reference(ops.a, ops.b, dtype, "DRELU", mask)
    d, none = run_backward(ops, "DRELU", mask, force_config=cfg, fused=fused)
    assert none is None and np.array_equal(d, exact_bits(dz, dtype))
    for layout in ("row", "col"):
        _, grad_ref, _ = eo.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, layout)
        d, grad = run_backward(ops, "DRELU_BGRAD", mask, layout, force_config=cfg, fused=fused)
        assert np.array_equal(d, exact_bits(dz, dtype))
        assert np.array_equal(grad, grad_ref), layout


def test_random_shapes_sweep():
    """24 seeded random cases on small-integer operands: m from 1 to 700, n
    and k multiples of 8 up to 720 and 1040; config, dtype, gradient axis,
    fused or two-kernel path, and DRELU or DRELU_BGRAD drawn at random.  The
    fp32 sums stay exact, so dZ is the single correct rounding and the fused
    gradient equals the oracle's bit for bit; the two-kernel path sums the
    rounded D, so its gradient is held to the bound that allows for that."""
    rng = np.random.default_rng(4242)
    for case in range(24):
        m = int(rng.integers(1, 701))
        n = 8 * int(rng.integers(1, 91))
        k = 8 * int(rng.integers(1, 131))
        dtype = ("fp16", "bf16")[int(rng.integers(2))]
        cfg = int(rng.integers(len(CONFIGS)))
        layout = ("row", "col")[int(rng.integers(2))]
        fused = bool(rng.integers(2))
        epilog = ("DRELU", "DRELU_BGRAD")[int(rng.integers(2))]
        tag = f"case {case}: {m}x{n}x{k} {dtype} {epilog} cfg={cfg} grad={layout} fused={fused}"
        print(tag, flush=True)
        ops = W.integer_operands(m, n, k, dtype, seed=900 + case, lo=-1, hi=1)
        mask = random_mask(m, n, 950 + case)
        dz, grad_ref, bound = eo.backward_reference(ops.a, ops.b, dtype, epilog, mask,
                                                    layout if epilog == "DRELU_BGRAD" else None)
        d, grad = run_backward(ops, epilog, mask, layout if epilog == "DRELU_BGRAD" else None,
                               force_config=cfg, fused=fused)
        bad = d != exact_bits(dz, dtype)
        assert not bad.any(), f"{tag}: {int(bad.sum())} outputs differ; first {tuple(np.argwhere(bad)[0])}"
        if epilog == "DRELU_BGRAD" and fused:
            assert np.array_equal(grad, grad_ref), f"{tag}: gradient differs"
        elif epilog == "DRELU_BGRAD":
            compare_bias_grad(grad, grad_ref, bound, d_ref=dz, dtype=dtype, layout=layout)
        else:
            assert grad is None


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_normal_within_bounds(dtype, cfg):
    m, n, k = 520, 392, 328
    ops = W.gemm_operands(m, n, k, dtype, seed=60 + cfg, a_std=0.7, b_std=1.0 / np.sqrt(k), bias_layout="col")
    mask = random_mask(m, n, 100 + cfg)
    for layout in ("row", "col"):
        dz, grad_ref, bound = eo.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, layout)
        d, grad = run_backward(ops, "DRELU_BGRAD", mask, layout, force_config=cfg)
        compare(d, dz, dtype)
        compare_bias_grad(grad, grad_ref, bound)
        d2, grad2 = run_backward(ops, "DRELU_BGRAD", mask, layout, force_config=cfg, fused=False)
        compare(d2, dz, dtype, unfused=True)
        compare_bias_grad(grad2, grad_ref, bound, d_ref=dz, dtype=dtype, layout=layout)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_forward_then_backward(dtype):
    """The chain a training step runs: forward RELU_AUX_BIAS, then the backward
    epilogue on its mask.  The oracle's own forward mask is the oracle input
    (and the backward's, checked against the oracle); the GPU's forward mask
    feeds a second backward run, which must agree with the first wherever the
    two masks agree and be zero wherever the GPU mask is 0.  No GPU output is
    ever an oracle input."""
    m, n, k = 264, 136, 200
    fwd = W.gemm_operands(m, n, k, dtype, seed=77, a_std=1.0, b_std=1.0 / np.sqrt(k), bias_layout="col",
                          bias_std=0.5)
    d_fwd, mask_gpu = run(fwd, "RELU_AUX_BIAS")
    y, z, mask_ref = eo.reference(fwd.a, fwd.b, dtype, "RELU_AUX_BIAS", fwd.bias, "col")
    compare(d_fwd, y, dtype, z=z, mask=mask_gpu, mask_ref=mask_ref)
    grad_ops = W.gemm_operands(m, n, 96, dtype, seed=78, a_std=0.7, b_std=1.0 / np.sqrt(96), bias_layout="col")
    dz, grad_ref, bound = eo.backward_reference(grad_ops.a, grad_ops.b, dtype, "DRELU_BGRAD", mask_ref, "col")
    d_ref_mask, grad = run_backward(grad_ops, "DRELU_BGRAD", mask_ref, "col")
    compare(d_ref_mask, dz, dtype)
    compare_bias_grad(grad, grad_ref, bound)
    d_gpu_mask, _ = run_backward(grad_ops, "DRELU_BGRAD", mask_gpu, "col")
    keep_gpu, keep_ref = eo.unpack_mask(mask_gpu, n), eo.unpack_mask(mask_ref, n)
    same = keep_gpu == keep_ref
    assert np.array_equal(d_gpu_mask[same], d_ref_mask[same])
    assert not eo.widen(d_gpu_mask, dtype)[~keep_gpu].any()


def test_edges_and_empty():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    for (m, n, k) in [(1, 8, 8), (33, 8, 16), (7, 24, 520), (40, 72, 0)]:
        for dtype in ("fp16", "bf16"):
            ops = W.gemm_operands(m, n, k, dtype, seed=m + n + k, a_std=1.0, bias_layout="col")
            mask = random_mask(m, n, m * n)
            for layout in ("row", "col"):
                dz, grad_ref, bound = eo.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, layout)
                if k == 0:
                    a = torch.empty((m, 0), dtype=torch.float16 if dtype == "fp16" else torch.bfloat16, device="cuda")
                    b = torch.empty((0, n), dtype=a.dtype, device="cuda")
                    g = torch.full((m, 1) if layout == "row" else (1, n), float("nan"), device="cuda")
                    with egm.Matmul(a, b) as mm:
                        mm.plan("DRELU_BGRAD", {"bias_grad": g})
                        d, grad = mm.execute(aux=torch.from_numpy(mask).cuda())
                    torch.cuda.synchronize()
                    assert not eo.widen(to_host_bits(d), dtype).any() and not grad.cpu().numpy().any()
                    continue
                d, grad = run_backward(ops, "DRELU_BGRAD", mask, layout)
                compare(d, dz, dtype)
                compare_bias_grad(grad, grad_ref, bound)
    # an empty m: the (1,n) gradient is a sum over no rows, all zeros
    a = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    b = torch.zeros((64, 16), dtype=torch.float16, device="cuda")
    g = torch.full((1, 16), float("nan"), device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("DRELU_BGRAD", {"bias_grad": g})
        d, grad = mm.execute(aux=torch.empty((0, 2), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert d.shape == (0, 16) and not grad.cpu().numpy().any()
    # an empty n: the (m,1) gradient is a sum over no columns, all zeros
    a = torch.ones((40, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((64, 0), dtype=torch.bfloat16, device="cuda")
    g = torch.full((40, 1), float("nan"), device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("DRELU_BGRAD", {"bias_grad": g})
        d, grad = mm.execute(aux=torch.empty((40, 0), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert d.shape == (40, 0) and grad.shape == (40, 1) and not grad.cpu().numpy().any()


def test_deterministic_gradient():
    ops = W.gemm_operands(1000, 520, 264, "bf16", seed=9, bias_layout="col")
    mask = random_mask(1000, 520, 5)
    _, g1 = run_backward(ops, "DRELU_BGRAD", mask, "col")
    _, g2 = run_backward(ops, "DRELU_BGRAD", mask, "col")
    assert np.array_equal(g1, g2)
