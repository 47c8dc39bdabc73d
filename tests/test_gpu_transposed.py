"""B given transposed ([n, k] row-major, a linear layer's weight) on the GPU
against the CPU oracle: the oracle takes B = W^T, the exact transpose of the
same bit patterns."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import bias_tensor, compare, exact_bits, fp8_to_device, run_backward, scale_tensor, to_device, to_host_bits

pytestmark = pytest.mark.gpu

CONFIGS = tuple(range(8))  # every tile config (5, 6, 7: 16x16x32 MFMA blocks)
FP8_CONFIGS = (0, 1, 2, 3, 4)  # the configs built for fp8 operands


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def _run_bt(ops, epilog, *, fused=True, force_config=-1):
    """ops.b is B [k, n]; the GPU gets W = B^T [n, k] contiguous and plans on W.t()."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = to_device(ops.a, ops.dtype)
    w = to_device(np.ascontiguousarray(ops.b.T), ops.dtype)
    ins = {}
    if epilog != "DEFAULT":
        ins["bias"] = bias_tensor(ops.bias, ops.bias_layout, ops.dtype)
    if epilog == "BIAS_RESIDUAL":
        ins["residual"] = to_device(ops.residual, ops.dtype)
    with egm.Matmul(a, w.t()) as mm:
        assert mm.bt
        mm.plan(epilog, ins, fused=fused, force_config=force_config)
        assert " b=[n,k]" in mm.describe()
        out = mm.execute()
        torch.cuda.synchronize()
    if isinstance(out, tuple):
        return to_host_bits(out[0]), out[1].cpu().numpy()
    return to_host_bits(out), None


@pytest.mark.parametrize("cfg", CONFIGS)
def test_residual_every_slab_count(cfg):
    """BIAS_RESIDUAL with B given transposed at every slab count from 1 to
    past two turns of the deepest ring, with and without a partial last slab,
    bit-exact on small-integer operands."""
    m, n = 72, 264
    for kt in range(1, 11):
        for k in (64 * kt, 64 * kt - 56):
            ops = W.integer_operands(m, n, k, "fp16", seed=300 * cfg + k, lo=-1, hi=1, bias_layout="col",
                                     residual=True)
            y, _, _ = eo.reference(ops.a, ops.b, "fp16", "BIAS_RESIDUAL", ops.bias, ops.bias_layout, ops.residual)
            d, _ = _run_bt(ops, "BIAS_RESIDUAL", force_config=cfg)
            assert np.array_equal(d, exact_bits(y, "fp16")), f"k={k}"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_integer_exact(dtype, cfg):
    m, n, k = 300, 264, 136
    ops = W.integer_operands(m, n, k, dtype, seed=cfg + 90, bias_layout="col" if cfg % 2 else "row", residual=True)
    for epilog in ("BIAS_RESIDUAL", "RELU_AUX_BIAS", "DEFAULT"):
        y, z, mref = eo.reference(ops.a, ops.b, dtype, epilog, ops.bias, ops.bias_layout, ops.residual)
        d, mask = _run_bt(ops, epilog, force_config=cfg)
        assert np.array_equal(d, exact_bits(y, dtype)), epilog
        if mref is not None:
            assert np.array_equal(mask, mref)
    y, _, _ = eo.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, ops.bias_layout)
    d, _ = _run_bt(ops, "BIAS", force_config=cfg, fused=False)
    compare(d, y, dtype, unfused=True)


@pytest.mark.parametrize("cfg", [0, 3, 4])
def test_normal_every_epilog(cfg):
    ops = W.gemm_operands(520, 392, 328, "bf16", seed=70 + cfg, a_std=1.0, b_std=0.4 / np.sqrt(328),
                          bias_layout="col", bias_std=0.3, residual_std=0.3)
    for epilog in ("DEFAULT", "BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL"):
        y, z, mref = eo.reference(ops.a, ops.b, "bf16", epilog, ops.bias, "col", ops.residual)
        d, mask = _run_bt(ops, epilog, force_config=cfg)
        compare(d, y, "bf16", z=z, mask=mask, mask_ref=mref)


@pytest.mark.parametrize("k", [144, 272])
@pytest.mark.parametrize("cfg", FP8_CONFIGS)
def test_fp8_pairs(cfg, k):
    """k = 144: two 128-deep k-slabs, the second ragged; k = 272: three, so
    the two-slab ring of config 0 ends on a slab after its main loop."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    for fa, fb in [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]:
        ops = W.fp8_integer_operands(304, 272, k, fa, fb, "bf16", seed=cfg + k, bias_layout="col", scale_a=0.5,
                                     scale_b=4.0)
        a = fp8_to_device(ops.a, fa)
        w = fp8_to_device(np.ascontiguousarray(ops.b.T), fb)
        with egm.Matmul(a, w.t(), scale_a=scale_tensor(ops.scale_a), scale_b=scale_tensor(ops.scale_b),
                        out_dtype=torch.bfloat16) as mm:
            mm.plan("RELU_AUX_BIAS", {"bias": bias_tensor(ops.bias, "col", "bf16")}, force_config=cfg)
            d, mask = mm.execute()
            torch.cuda.synchronize()
        y, z, mref = eo.reference_fp8(ops.a, ops.b, fa, fb, ops.scale_a, ops.scale_b, "bf16", "RELU_AUX_BIAS",
                                      ops.bias, "col")
        assert np.array_equal(to_host_bits(d), exact_bits(y, "bf16")), (fa, fb)
        assert np.array_equal(mask.cpu().numpy(), mref)


def test_random_shapes_sweep():
    """Seeded random cases with B given transposed, bit-exact on small-integer
    operands: 24 in 16 bits (m 1..700, n and k multiples of 8 up to 720 and
    1040, every config) and 16 in fp8 (n and k multiples of 16, the fp8
    configs, every format pair, power-of-two scales)."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    rng = np.random.default_rng(4242)
    epilogs = ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL")
    for case in range(24):
        m, n, k = int(rng.integers(1, 701)), 8 * int(rng.integers(1, 91)), 8 * int(rng.integers(1, 131))
        dtype = ("fp16", "bf16")[int(rng.integers(2))]
        epilog = epilogs[int(rng.integers(len(epilogs)))]
        cfg = CONFIGS[int(rng.integers(len(CONFIGS)))]
        layout = ("row", "col")[int(rng.integers(2))]
        tag = f"case {case}: {m}x{n}x{k} {dtype} {epilog} cfg={cfg} bias={layout}"
        print(tag, flush=True)
        ops = W.integer_operands(m, n, k, dtype, seed=700 + case, bias_layout=layout, residual=True)
        y, z, mref = eo.reference(ops.a, ops.b, dtype, epilog, None if epilog == "DEFAULT" else ops.bias,
                                  None if epilog == "DEFAULT" else layout, ops.residual)
        d, mask = _run_bt(ops, epilog, force_config=cfg)
        bad = d != exact_bits(y, dtype)
        assert not bad.any(), f"{tag}: {int(bad.sum())} outputs differ; first {tuple(np.argwhere(bad)[0])}"
        if mref is not None:
            assert np.array_equal(mask, mref), f"{tag}: mask differs"
    pairs = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
    for case in range(16):
        m, n, k = int(rng.integers(1, 601)), 16 * int(rng.integers(1, 41)), 16 * int(rng.integers(1, 65))
        fa, fb = pairs[int(rng.integers(4))]
        out = ("fp16", "bf16")[int(rng.integers(2))]
        cfg = FP8_CONFIGS[int(rng.integers(len(FP8_CONFIGS)))]
        layout = ("row", "col")[int(rng.integers(2))]
        tag = f"fp8 case {case}: {m}x{n}x{k} {fa}x{fb}->{out} cfg={cfg} bias={layout}"
        print(tag, flush=True)
        ops = W.fp8_integer_operands(m, n, k, fa, fb, out, seed=800 + case, bias_layout=layout, scale_a=2.0,
                                     scale_b=0.5)
        a = fp8_to_device(ops.a, fa)
        w = fp8_to_device(np.ascontiguousarray(ops.b.T), fb)
        tdt = torch.float16 if out == "fp16" else torch.bfloat16
        with egm.Matmul(a, w.t(), scale_a=scale_tensor(ops.scale_a), scale_b=scale_tensor(ops.scale_b),
                        out_dtype=tdt) as mm:
            mm.plan("RELU_AUX_BIAS", {"bias": bias_tensor(ops.bias, layout, out)}, force_config=cfg)
            d, mask = mm.execute()
            torch.cuda.synchronize()
        y, z, mref = eo.reference_fp8(ops.a, ops.b, fa, fb, ops.scale_a, ops.scale_b, out, "RELU_AUX_BIAS",
                                      ops.bias, layout)
        bad = to_host_bits(d) != exact_bits(y, out)
        assert not bad.any(), f"{tag}: {int(bad.sum())} outputs differ"
        assert np.array_equal(mask.cpu().numpy(), mref), f"{tag}: mask differs"


def test_backward_and_strided_batch():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k = 200, 144, 136
    ops = W.integer_operands(m, n, k, "fp16", seed=5)
    mask = np.random.default_rng(3).integers(0, 256, size=(m, n // 8), dtype=np.uint8)
    a = to_device(ops.a, "fp16")
    w = to_device(np.ascontiguousarray(ops.b.T), "fp16")
    grad = torch.full((1, n), float("nan"), dtype=torch.float32, device="cuda")
    with egm.Matmul(a, w.t()) as mm:
        mm.plan("DRELU_BGRAD", {"bias_grad": grad})
        d, g = mm.execute(aux=torch.from_numpy(mask).cuda())
        torch.cuda.synchronize()
    dz, gref, _ = eo.backward_reference(ops.a, ops.b, "fp16", "DRELU_BGRAD", mask, "col")
    assert np.array_equal(to_host_bits(d), exact_bits(dz, "fp16"))
    assert np.array_equal(g.double().cpu().numpy().reshape(-1), gref)
    # a batch of inputs through one weight, and a batch of weights
    a_list = [W.integer_bits((m, k), -2, 2, "fp16", 11, z) for z in range(3)]
    w_list = [W.integer_bits((n, k), -2, 2, "fp16", 12, z) for z in range(3)]
    a_b = torch.stack([to_device(x, "fp16") for x in a_list])
    w_b = torch.stack([to_device(x, "fp16") for x in w_list])  # [batch, n, k] contiguous
    with egm.Matmul(a, w.t()) as mm:
        mm.plan("DEFAULT")
        d1 = mm.execute_batched(a_b, w.t())
        d2 = mm.execute_batched(a, w_b.transpose(1, 2))
        torch.cuda.synchronize()
    for z in range(3):
        y1, _, _ = eo.reference(a_list[z], ops.b, "fp16", "DEFAULT")
        y2, _, _ = eo.reference(ops.a, np.ascontiguousarray(w_list[z].T), "fp16", "DEFAULT")
        assert np.array_equal(to_host_bits(d1[z]), exact_bits(y1, "fp16"))
        assert np.array_equal(to_host_bits(d2[z]), exact_bits(y2, "fp16"))


def test_linear_layer_usage():
    """y = relu(x W^T + b) with W stored [out, in], as a linear layer holds it."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    x_bits = W.normal_bits((256, 512), 1.0, "bf16", 21, 0)
    w_bits = W.normal_bits((384, 512), 0.4 / np.sqrt(512), "bf16", 21, 1)
    b_bits = W.normal_bits((384,), 0.3, "bf16", 21, 2)
    x, w = to_device(x_bits, "bf16"), to_device(w_bits, "bf16")
    with egm.Matmul(x, w.t()) as mm:
        mm.plan("RELU_BIAS", {"bias": to_device(b_bits, "bf16").reshape(1, -1)})
        y = mm.execute()
        torch.cuda.synchronize()
    yr, _, _ = eo.reference(x_bits, np.ascontiguousarray(w_bits.T), "bf16", "RELU_BIAS", b_bits, "col")
    compare(to_host_bits(y), yr, "bf16")
