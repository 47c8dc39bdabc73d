"""HIP path vs the CPU oracle, element by element (GPU: MI355X / gfx950).

Every call goes through the C ABI (thin Python binding over libegm.so).
Shapes span several tiles of every config with ragged tails in m, n and k.
"""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import compare, exact_bits, run, to_device, to_host_bits

pytestmark = pytest.mark.gpu

EPILOGS_EXACT = ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL")
ALL_EPILOGS = EPILOGS_EXACT + ("GELU_BIAS",)
CONFIGS = tuple(range(8))  # every tile config (5, 6, 7: 16x16x32 MFMA blocks)
RAGGED = (300, 264, 136)  # m = 256+44, n = 256+8, k = 2*64+8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def oracle_for(ops, epilog, rows=None):
    return eo.reference(ops.a, ops.b, ops.dtype, epilog,
                        None if epilog == "DEFAULT" else ops.bias,
                        None if epilog == "DEFAULT" else ops.bias_layout,
                        ops.residual if epilog == "BIAS_RESIDUAL" else None, rows=rows)


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("epilog", EPILOGS_EXACT)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_integer_exact_bits(dtype, epilog, cfg):
    """Small-integer operands: fp32 accumulation is exact, so D must equal the
    single correct rounding of the exact result bit for bit, and the mask must
    equal (Z > 0) everywhere, Z = 0 included."""
    m, n, k = RAGGED
    layout = "col" if (cfg + len(epilog)) % 2 else "row"
    ops = W.integer_operands(m, n, k, dtype, seed=cfg, bias_layout=layout, residual=True)
    d, mask = run(ops, epilog, force_config=cfg)
    y, z, mref = oracle_for(ops, epilog)
    want = exact_bits(y, dtype)
    bad = d != want
    assert not bad.any(), f"{int(bad.sum())} outputs differ; first {tuple(np.argwhere(bad)[0])}"
    if epilog == "RELU_AUX_BIAS":
        assert np.array_equal(mask, mref)
        assert (z == 0).any()  # the strict predicate is exercised


@pytest.mark.parametrize("cfg", CONFIGS)
def test_ring_turns_and_partial_slab(cfg):
    """The main loop runs whole turns of its ring of k-slabs, then the slabs
    left over, and skips the A copies' per-lane k check in slabs wholly below
    K: every count of 64-deep slabs from 1 to past two turns of the deepest
    ring (4), with and without a partial last slab, bit-exact on
    small-integer operands, with the mask epilogue and with the residual."""
    m, n = 72, 264
    for kt in range(1, 11):
        for k in (64 * kt, 64 * kt - 56):
            ops = W.integer_operands(m, n, k, "bf16", seed=100 * cfg + k, lo=-1, hi=1, bias_layout="row",
                                     residual=True)
            for epilog in ("RELU_AUX_BIAS", "BIAS_RESIDUAL"):
                d, mask = run(ops, epilog, force_config=cfg)
                y, z, mref = oracle_for(ops, epilog)
                bad = d != exact_bits(y, "bf16")
                assert not bad.any(), (f"{epilog} k={k}: {int(bad.sum())} outputs differ; "
                                       f"first {tuple(np.argwhere(bad)[0])}")
                if epilog == "RELU_AUX_BIAS":
                    assert np.array_equal(mask, mref), f"k={k}: mask differs"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("epilog", ALL_EPILOGS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_normal_within_tolerance(dtype, epilog, cfg):
    m, n, k = 520, 392, 328
    layout = "row" if cfg % 2 else "col"
    # |Y| stays far below 8, where half a bf16 ulp (1/32) would exceed 2e-2
    ops = W.gemm_operands(m, n, k, dtype, seed=10 + cfg, a_std=0.7, b_std=1.0 / np.sqrt(k),
                          bias_layout=layout, bias_std=0.5, residual_std=0.5)
    d, mask = run(ops, epilog, force_config=cfg)
    y, z, mref = oracle_for(ops, epilog)
    compare(d, y, dtype, z=z, mask=mask, mask_ref=mref)


def test_random_shapes_sweep():
    """48 seeded random cases, bit-exact on small-integer operands: m from 1
    to 700, n and k multiples of 8 up to 720 and 1040, every config, dtype,
    bias layout and exact epilogue drawn at random (fp32 sums stay exact, so
    D is the single correct rounding of the exact result whatever the shape)."""
    rng = np.random.default_rng(2024)
    for case in range(48):
        m = int(rng.integers(1, 701))
        n = 8 * int(rng.integers(1, 91))
        k = 8 * int(rng.integers(1, 131))
        dtype = ("fp16", "bf16")[int(rng.integers(2))]
        epilog = EPILOGS_EXACT[int(rng.integers(len(EPILOGS_EXACT)))]
        cfg = int(rng.integers(len(CONFIGS)))
        layout = ("row", "col")[int(rng.integers(2))]
        tag = f"case {case}: {m}x{n}x{k} {dtype} {epilog} cfg={cfg} bias={layout}"
        print(tag, flush=True)
        ops = W.integer_operands(m, n, k, dtype, seed=500 + case, bias_layout=layout, residual=True)
        d, mask = run(ops, epilog, force_config=cfg)
        y, z, mref = oracle_for(ops, epilog)
        bad = d != exact_bits(y, dtype)
        assert not bad.any(), f"{tag}: {int(bad.sum())} outputs differ; first {tuple(np.argwhere(bad)[0])}"
        if epilog == "RELU_AUX_BIAS":
            assert np.array_equal(mask, mref), f"{tag}: mask differs"


@pytest.mark.parametrize("epilog", ["BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_unfused_path(dtype, epilog):
    m, n, k = 264, 520, 200
    ops = W.gemm_operands(m, n, k, dtype, seed=3, a_std=0.7, b_std=1.0 / np.sqrt(k),
                          bias_layout="row" if dtype == "fp16" else "col", bias_std=0.5, residual_std=0.5)
    d, mask = run(ops, epilog, fused=False)
    y, z, mref = oracle_for(ops, epilog)
    compare(d, y, dtype, z=z, mask=mask, mask_ref=mref, unfused=True)


def test_mask_bit_order_and_placement():
    """Z[i,j] = j - i: bit j%8 of byte j/8 in row i is set iff j > i."""
    m, n = 72, 80
    for dtype in ("fp16", "bf16"):
        a = eo.round_to_bits(np.stack([np.ones(m), np.arange(m)], axis=1), dtype)
        a = np.concatenate([a, np.zeros((m, 6), np.uint16)], axis=1)  # k = 8
        b = eo.round_to_bits(np.stack([np.arange(n), -np.ones(n)], axis=0), dtype)
        b = np.concatenate([b, np.zeros((6, n), np.uint16)], axis=0)
        ops = W.Operands(m, n, 8, dtype, a, b, np.zeros(n, np.uint16), "col")
        for cfg in CONFIGS:
            d, mask = run(ops, "RELU_AUX_BIAS", force_config=cfg)
            want = np.array([[sum(1 << t for t in range(8) if 8 * c + t > i) for c in range(n // 8)]
                             for i in range(m)], dtype=np.uint8)
            assert np.array_equal(mask, want), (dtype, cfg)
            dd = eo.widen(d, dtype)
            assert np.array_equal(dd, np.maximum(np.arange(n)[None, :] - np.arange(m)[:, None], 0))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_identity_and_zero_operands(dtype):
    k, n = 136, 264
    ops = W.gemm_operands(k, n, k, dtype, seed=5, bias_layout="row")
    ops.a = eo.round_to_bits(np.eye(k), dtype)
    d, _ = run(ops, "BIAS")
    assert np.array_equal(d, eo.round_to_bits(eo.widen(ops.b, dtype) + eo.widen(ops.bias, dtype)[:, None], dtype))
    ops.b = np.zeros_like(ops.b)
    d, _ = run(ops, "BIAS")
    assert np.array_equal(d, np.repeat(ops.bias[:, None], n, axis=1))
    # zero bias is the plain product
    ops = W.gemm_operands(200, 136, 96, dtype, seed=6, bias_layout="col")
    ops.bias = np.zeros_like(ops.bias)
    d0, _ = run(ops, "DEFAULT")
    d1, _ = run(ops, "BIAS")
    assert np.array_equal(d0, d1)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_relu_invariants_and_gelu_odd_part(dtype):
    ops = W.gemm_operands(264, 136, 72, dtype, seed=7, a_std=1.0, b_std=0.2, bias_layout="col")
    d, mask = run(ops, "RELU_AUX_BIAS")
    dd = eo.widen(d, dtype)
    assert (dd >= 0).all()
    assert int(np.unpackbits(mask).sum()) == int((dd > 0).sum())
    # gelu(z) - gelu(-z) = z with zero bias: D(A) - D(-A) = A.B
    ops.bias = np.zeros_like(ops.bias)
    d_pos, _ = run(ops, "GELU_BIAS")
    neg = ops.a ^ np.uint16(0x8000)
    ops_neg = W.Operands(ops.m, ops.n, ops.k, dtype, neg, ops.b, ops.bias, "col")
    d_neg, _ = run(ops_neg, "GELU_BIAS")
    p = eo.widen(ops.a, dtype) @ eo.widen(ops.b, dtype)
    diff = eo.widen(d_pos, dtype) - eo.widen(d_neg, dtype)
    assert np.abs(diff - p).max() <= 2 * eo.TOLERANCE[dtype]


def test_edge_shapes():
    # one row, one 8-column group
    for dtype in ("fp16", "bf16"):
        for (m, n, k) in [(1, 8, 8), (1, 8, 64), (33, 8, 8), (7, 24, 520), (513, 8, 16)]:
            ops = W.gemm_operands(m, n, k, dtype, seed=m + n + k, a_std=1.0, bias_layout="row", residual_std=1.0)
            for ep in ("BIAS_RESIDUAL", "RELU_AUX_BIAS"):
                d, mask = run(ops, ep)
                y, z, mref = oracle_for(ops, ep)
                compare(d, y, dtype, z=z, mask=mask, mask_ref=mref)


def test_k_zero_gives_epilogue_of_bias():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n = 40, 24
    bias = W.normal_bits((n,), 1.0, "fp16", 0, 2)
    a = torch.empty((m, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, n), dtype=torch.float16, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": to_device(bias, "fp16").reshape(1, n)})
        d, mask = mm.execute()
    torch.cuda.synchronize()
    bb = eo.widen(bias, "fp16")
    assert np.array_equal(eo.widen(to_host_bits(d), "fp16"), np.repeat(np.maximum(bb, 0)[None, :], m, axis=0))
    assert np.array_equal(mask.cpu().numpy(), np.repeat(np.packbits(bb > 0, bitorder="little")[None, :], m, axis=0))


def test_empty_m_is_noop():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    b = torch.zeros((64, 16), dtype=torch.float16, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("BIAS", {"bias": torch.zeros((1, 16), dtype=torch.float16, device="cuda")})
        d = mm.execute()
    torch.cuda.synchronize()
    assert d.shape == (0, 16)


def test_empty_n_is_noop():
    """n = 0: D and the mask are empty; nothing is launched and the mask may be
    the empty tensor."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = torch.ones((40, 64), dtype=torch.float16, device="cuda")
    b = torch.empty((64, 0), dtype=torch.float16, device="cuda")
    for epilog, ins in (("BIAS", {"bias": torch.zeros((40, 1), dtype=torch.float16, device="cuda")}),
                        ("RELU_AUX_BIAS", {"bias": torch.zeros((40, 1), dtype=torch.float16, device="cuda")}),
                        ("DEFAULT", {})):
        with egm.Matmul(a, b) as mm:
            mm.plan(epilog, ins)
            out = mm.execute()
        torch.cuda.synchronize()
        d = out[0] if isinstance(out, tuple) else out
        assert d.shape == (40, 0), epilog
        if isinstance(out, tuple):
            assert out[1].shape == (40, 0)


@pytest.mark.slow
def test_maximum_n_and_k():
    """n = 2^21 with one row, and k = 2^21 with a single 8x8 output."""
    for (m, n, k) in [(3, 1 << 21, 16), (8, 8, 1 << 21)]:
        ops = W.gemm_operands(m, n, k, "bf16", seed=1, bias_layout="col", residual_std=1.0)
        d, mask = run(ops, "RELU_AUX_BIAS")
        y, z, mref = oracle_for(ops, "RELU_AUX_BIAS")
        compare(d, y, "bf16", z=z, mask=mask, mask_ref=mref)


@pytest.mark.slow
def test_maximum_m_row_bias():
    """m = 2^30 + 200 rows, n = k = 8, (m,1) bias, RELU_AUX_BIAS: rows past
    2^30 sit more than 2^31 bytes into the bias, and the 64x64 tile's grid
    would exceed 2^32 - 1 work-items.  A repeats a seeded 4096-row block (tiled
    on the device by torch); the bias is a full seeded draw.  The oracle runs
    on the sub-problem of sampled rows: every row across the 2^30 boundary,
    the first and last 256 and 2048 random ones."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, blk = (1 << 30) + 200, 8, 8, 4096
    ops = W.gemm_operands(blk, n, k, "fp16", seed=5, bias_layout="row")
    bias_bits = W.normal_bits((m,), 1.0, "fp16", seed=5, tensor_index=7)
    g = np.random.default_rng(3)
    rows = np.unique(np.concatenate([
        np.arange(256), np.arange((1 << 30) - 256, m), g.integers(256, (1 << 30) - 256, 2048)])).astype(np.int64)
    a = to_device(ops.a, "fp16").repeat(m // blk + 1, 1)[:m]
    b = to_device(ops.b, "fp16")
    bias = to_device(bias_bits, "fp16").reshape(-1, 1)
    sel = torch.from_numpy(rows).cuda()
    y, z, mref = eo.reference(ops.a[rows % blk], ops.b, "fp16", "RELU_AUX_BIAS", bias_bits[rows], "row")
    with egm.Matmul(a, b) as mm:
        with pytest.raises(egm.EgmError):
            mm.plan("RELU_AUX_BIAS", {"bias": bias}, force_config=4)  # 64x64: grid too large
        for cfg in (-1, 0, 3):
            print(f"[maximum m={m} cfg={cfg}]", flush=True)
            mm.plan("RELU_AUX_BIAS", {"bias": bias}, force_config=cfg)
            d, mask = mm.execute()
            ds, ms = to_host_bits(d.index_select(0, sel)), mask.index_select(0, sel).cpu().numpy()
            del d, mask
            compare(ds, y, "fp16", z=z, mask=ms, mask_ref=mref)


def test_determinism_and_stream():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    ops = W.gemm_operands(1000, 520, 264, "bf16", seed=9, bias_layout="col")
    a, b = to_device(ops.a, "bf16"), to_device(ops.b, "bf16")
    bias = to_device(ops.bias, "bf16").reshape(1, -1)
    s = torch.cuda.Stream()
    with egm.Matmul(a, b) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": bias})
        d1, m1 = mm.execute()
        with torch.cuda.stream(s):
            d2, m2 = mm.execute()
        torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(m1, m2)
    # the stream argument: outputs are allocated on that stream and a plan's
    # workspace (two-kernel path) is recorded on it
    with egm.Matmul(a, b) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": bias}, fused=False)
        d3, m3 = mm.execute()
        torch.cuda.synchronize()
        d4, m4 = mm.execute(stream=s)
        s.synchronize()
    assert torch.equal(d3, d4) and torch.equal(m3, m4)
    y, z, mref = oracle_for(ops, "RELU_AUX_BIAS")
    compare(to_host_bits(d4), y, "bf16", z=z, mask=m4.cpu().numpy(), mask_ref=mref, unfused=True)


def test_wrapper_rejects_bad_inputs():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = torch.zeros(64, 32, dtype=torch.float16, device="cuda")
    b = torch.zeros(32, 16, dtype=torch.float16, device="cuda")
    mm = egm.Matmul(a, b)
    with pytest.raises(ValueError):
        mm.plan("BIAS", {"bias": torch.zeros(64, dtype=torch.float16, device="cuda")})  # 1-D: not (m,1)/(1,n)
    with pytest.raises(ValueError):
        mm.plan("BIAS", {"bias": torch.zeros(16, 1, dtype=torch.float16, device="cuda")})
    with pytest.raises(TypeError):
        mm.plan("BIAS", {"bias": torch.zeros(64, 1, dtype=torch.bfloat16, device="cuda")})
    with pytest.raises(TypeError):
        egm.Matmul(a, b.to(torch.bfloat16))
    with pytest.raises(RuntimeError):
        mm.execute()
    mm.free()
