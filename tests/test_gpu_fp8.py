"""fp8 operands (OCP E4M3 / E5M2, per-tensor scales, 16-bit bias / residual /
output) on the GPU against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import compare, exact_bits, run_fp8

pytestmark = pytest.mark.gpu

CONFIGS = (0, 1, 2, 3, 4)  # the configs built for fp8 operands (32x32x64 MFMA blocks)
PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
FORWARD = ("DEFAULT", "BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL")
# product, bias and residual stds that keep |Y| well below 4, where bf16's half
# ulp (2^-7 .. 2^-6) stays inside the 2e-2 tolerance; from 8 up it is 2^-5
SMALL = dict(a_std=1.0, bias_std=0.3, residual_std=0.3)


def _b_std(k, v=0.4):
    return v / np.sqrt(k)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def _ref(ops, epilog):
    return eo.reference_fp8(ops.a, ops.b, ops.a_fmt, ops.b_fmt, ops.scale_a, ops.scale_b, ops.out_dtype, epilog,
                            ops.bias, ops.bias_layout, ops.residual)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_residual_every_slab_count(cfg):
    """fp8 slabs are 128 deep: every slab count from 1 to past two turns of
    the deepest ring (4), with and without a partial last slab, BIAS_RESIDUAL
    bit-exact on small-integer operands."""
    for kt in range(1, 11):
        for k in (128 * kt, 128 * kt - 112):
            ops = W.fp8_integer_operands(72, 272, k, "e4m3", "e4m3", "bf16", seed=40 * cfg + k,
                                         bias_layout="col", scale_a=2.0, scale_b=0.25, residual=True)
            y, _, _ = _ref(ops, "BIAS_RESIDUAL")
            d, _ = run_fp8(ops, "BIAS_RESIDUAL", force_config=cfg)
            assert np.array_equal(d, exact_bits(y, "bf16")), f"k={k}"


@pytest.mark.parametrize("out", ["fp16", "bf16"])
@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("pair", PAIRS, ids=["x".join(p) for p in PAIRS])
def test_integer_exact(pair, cfg, out):
    """Small integers, power-of-two scales: every step is exact in fp32, so D
    is the single correct rounding of the exact result, bit for bit (fused);
    the two-kernel path rounds twice and is held to the tolerance."""
    fa, fb = pair
    ops = W.fp8_integer_operands(300, 272, 144, fa, fb, out, seed=cfg + 7, bias_layout="row" if cfg % 2 else "col",
                                 scale_a=2.0, scale_b=0.25, residual=True)
    for epilog in ("BIAS_RESIDUAL", "RELU_AUX_BIAS", "DEFAULT"):
        y, z, mref = _ref(ops, epilog)
        d, mask = run_fp8(ops, epilog, force_config=cfg)
        assert np.array_equal(d, exact_bits(y, out)), epilog
        if mref is not None:
            assert np.array_equal(mask, mref)
    y, z, _ = _ref(ops, "BIAS")
    d, _ = run_fp8(ops, "BIAS", force_config=cfg, fused=False)
    compare(d, y, out, unfused=True)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_normal_every_epilog(cfg):
    ops = W.fp8_operands(520, 400, 336, "e4m3", "e4m3", "bf16", seed=20 + cfg, bias_layout="col", b_std=_b_std(336),
                         **SMALL)
    for epilog in FORWARD:
        y, z, mref = _ref(ops, epilog)
        d, mask = run_fp8(ops, epilog, force_config=cfg)
        st = compare(d, y, "bf16", z=z, mask=mask, mask_ref=mref)
        print(f"[fp8 e4m3 cfg={cfg} {epilog}] {st}", flush=True)


@pytest.mark.parametrize("out", ["fp16", "bf16"])
@pytest.mark.parametrize("pair", PAIRS, ids=["x".join(p) for p in PAIRS])
def test_normal_format_pairs(pair, out):
    fa, fb = pair
    ops = W.fp8_operands(392, 528, 464, fa, fb, out, seed=31, bias_layout="row", b_std=_b_std(464), **SMALL)
    for cfg in CONFIGS:
        for epilog in ("BIAS", "GELU_BIAS", "RELU_AUX_BIAS"):
            y, z, mref = _ref(ops, epilog)
            d, mask = run_fp8(ops, epilog, force_config=cfg)
            compare(d, y, out, z=z, mask=mask, mask_ref=mref)
        y, z, _ = _ref(ops, "BIAS_RESIDUAL")
        d, _ = run_fp8(ops, "BIAS_RESIDUAL", force_config=cfg, fused=False)
        compare(d, y, out, unfused=True)


def test_random_shapes_sweep():
    """32 seeded random fp8 cases, bit-exact on small-integer operands with
    power-of-two scales: m from 1 to 600, n and k multiples of 16 up to 640
    and 1024, every fp8 config, format pair, output dtype, bias layout and
    exact epilogue drawn at random."""
    rng = np.random.default_rng(808)
    epilogs = ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL")
    for case in range(32):
        m = int(rng.integers(1, 601))
        n = 16 * int(rng.integers(1, 41))
        k = 16 * int(rng.integers(1, 65))
        fa, fb = PAIRS[int(rng.integers(len(PAIRS)))]
        out = ("fp16", "bf16")[int(rng.integers(2))]
        epilog = epilogs[int(rng.integers(len(epilogs)))]
        cfg = CONFIGS[int(rng.integers(len(CONFIGS)))]
        layout = ("row", "col")[int(rng.integers(2))]
        tag = f"case {case}: {m}x{n}x{k} {fa}x{fb}->{out} {epilog} cfg={cfg} bias={layout}"
        print(tag, flush=True)
        ops = W.fp8_integer_operands(m, n, k, fa, fb, out, seed=900 + case, bias_layout=layout, scale_a=0.5,
                                     scale_b=2.0, residual=True)
        y, z, mref = _ref(ops, epilog)
        d, mask = run_fp8(ops, epilog, force_config=cfg)
        bad = d != exact_bits(y, out)
        assert not bad.any(), f"{tag}: {int(bad.sum())} outputs differ; first {tuple(np.argwhere(bad)[0])}"
        if mref is not None:
            assert np.array_equal(mask, mref), f"{tag}: mask differs"


def test_edges_null_scales_and_k0():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    from parity import bias_tensor, fp8_to_device, scale_tensor, to_host_bits
    for (m, n, k) in [(1, 16, 16), (33, 16, 32), (7, 48, 528), (300, 16, 16)]:
        ops = W.fp8_operands(m, n, k, "e5m2", "e4m3", "fp16", seed=m + n + k, bias_layout="col")
        y, z, mref = _ref(ops, "RELU_AUX_BIAS")
        d, mask = run_fp8(ops, "RELU_AUX_BIAS")
        compare(d, y, "fp16", z=z, mask=mask, mask_ref=mref)
    # NULL scales read as 1 (integer operands: raw fp8 values, exact results)
    ops = W.fp8_integer_operands(64, 80, 96, "e4m3", "e4m3", "bf16", seed=5, bias_layout="row")
    y1, _, _ = eo.reference_fp8(ops.a, ops.b, "e4m3", "e4m3", 1.0, 1.0, "bf16", "BIAS", ops.bias, "row")
    d, _ = run_fp8(ops, "BIAS", null_scales=True)
    assert np.array_equal(d, exact_bits(y1, "bf16"))
    # k = 0: D = epilogue(bias)
    a = torch.empty((40, 0), dtype=torch.float8_e4m3fn, device="cuda")
    b = torch.empty((0, 32), dtype=torch.float8_e4m3fn, device="cuda")
    bias_bits = W.normal_bits((32,), 1.0, "bf16", 3, 2)
    with egm.Matmul(a, b, scale_a=scale_tensor(3.0), out_dtype=torch.bfloat16) as mm:
        mm.plan("RELU_BIAS", {"bias": bias_tensor(bias_bits, "col", "bf16")})
        d = mm.execute()
        torch.cuda.synchronize()
    want = np.repeat(np.maximum(eo.widen(bias_bits, "bf16"), 0)[None, :], 40, axis=0)
    assert np.array_equal(eo.widen(to_host_bits(d), "bf16"), want)
    # empty m
    a = torch.empty((0, 32), dtype=torch.float8_e5m2, device="cuda")
    b = torch.zeros((32, 16), dtype=torch.float8_e5m2, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("DEFAULT")
        d = mm.execute()
        torch.cuda.synchronize()
    assert d.shape == (0, 16)


def test_scales_are_read_at_execute():
    """The plan binds the scale pointers; a new value written to them on the
    stream is used by the next execute without planning again."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    from parity import bias_tensor, fp8_to_device, scale_tensor, to_host_bits
    ops = W.fp8_operands(128, 96, 160, "e4m3", "e5m2", "fp16", seed=9, bias_layout="col")
    sa, sb = scale_tensor(ops.scale_a), scale_tensor(ops.scale_b)
    a, b = fp8_to_device(ops.a, "e4m3"), fp8_to_device(ops.b, "e5m2")
    with egm.Matmul(a, b, scale_a=sa, scale_b=sb, out_dtype=torch.float16) as mm:
        mm.plan("BIAS", {"bias": bias_tensor(ops.bias, "col", "fp16")})
        d1 = mm.execute()
        sa.mul_(4.0)
        d2 = mm.execute()
        torch.cuda.synchronize()
    y1, _, _ = eo.reference_fp8(ops.a, ops.b, "e4m3", "e5m2", ops.scale_a, ops.scale_b, "fp16", "BIAS", ops.bias, "col")
    y2, _, _ = eo.reference_fp8(ops.a, ops.b, "e4m3", "e5m2", np.float32(ops.scale_a * 4), ops.scale_b, "fp16", "BIAS",
                                ops.bias, "col")
    compare(to_host_bits(d1), y1, "fp16")
    compare(to_host_bits(d2), y2, "fp16")
