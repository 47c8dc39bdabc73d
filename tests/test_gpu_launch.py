"""Launch amortisation on the GPU: strided batches (one launch over many
problems) against the CPU oracle, and executes captured in a HIP graph whose
replays must reproduce the eager results bit for bit."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import bias_tensor, compare, fp8_to_device, scale_tensor, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def _stack(arrs, dtype):
    import torch
    return torch.stack([to_device(a, dtype) for a in arrs])


@pytest.mark.parametrize("cfg", list(range(8)))
def test_strided_batch_shared_weight(cfg):
    """Five problems with their own A and one shared B (a weight), RELU_AUX_BIAS."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype, batch = 304, 272, 136, "bf16", 5  # ragged for every tile; each mask 16-byte aligned
    base = W.gemm_operands(m, n, k, dtype, seed=50 + cfg, bias_layout="col")
    a_list = [W.normal_bits((m, k), 1.0 / np.sqrt(k), dtype, 60 + cfg, z) for z in range(batch)]
    with egm.Matmul(to_device(a_list[0], dtype), to_device(base.b, dtype)) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": bias_tensor(base.bias, "col", dtype)}, force_config=cfg)
        d, mask = mm.execute_batched(_stack(a_list, dtype), to_device(base.b, dtype))
        torch.cuda.synchronize()
    assert d.shape == (batch, m, n) and mask.shape == (batch, m, n // 8)
    for z in range(batch):
        y, zz, mref = eo.reference(a_list[z], base.b, dtype, "RELU_AUX_BIAS", base.bias, "col")
        compare(to_host_bits(d[z]), y, dtype, z=zz, mask=mask[z].cpu().numpy(), mask_ref=mref)


def test_strided_batch_random_sweep():
    """16 seeded random batches, bit-exact on small-integer operands: batch
    1..6, m 1..300, n and k multiples of 8 up to 320 and 520, config, dtype,
    bias layout and epilog (DEFAULT, BIAS, RELU_BIAS) at random, with A per
    problem and B either per problem or shared."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    from parity import exact_bits
    rng = np.random.default_rng(31)
    for case in range(16):
        batch = int(rng.integers(1, 7))
        m = int(rng.integers(1, 301))
        n = 8 * int(rng.integers(1, 41))
        k = 8 * int(rng.integers(1, 66))
        dtype = ("fp16", "bf16")[int(rng.integers(2))]
        cfg = int(rng.integers(8))
        layout = ("row", "col")[int(rng.integers(2))]
        epilog = ("DEFAULT", "BIAS", "RELU_BIAS")[int(rng.integers(3))]
        shared_b = bool(rng.integers(2))
        tag = f"case {case}: batch {batch} {m}x{n}x{k} {dtype} {epilog} cfg={cfg} bias={layout} shared_b={shared_b}"
        print(tag, flush=True)
        probs = [W.integer_operands(m, n, k, dtype, seed=2000 + 10 * case + z, bias_layout=layout) for z in range(batch)]
        bias = probs[0].bias
        b_list = [probs[0].b] * batch if shared_b else [p.b for p in probs]
        ins = {} if epilog == "DEFAULT" else {"bias": bias_tensor(bias, layout, dtype)}
        with egm.Matmul(to_device(probs[0].a, dtype), to_device(b_list[0], dtype)) as mm:
            mm.plan(epilog, ins, force_config=cfg)
            d = mm.execute_batched(_stack([p.a for p in probs], dtype),
                                   to_device(b_list[0], dtype) if shared_b else _stack(b_list, dtype))
            torch.cuda.synchronize()
        assert d.shape == (batch, m, n), tag
        for z in range(batch):
            y, _, _ = eo.reference(probs[z].a, b_list[z], dtype, epilog, None if epilog == "DEFAULT" else bias,
                                   None if epilog == "DEFAULT" else layout)
            bad = to_host_bits(d[z]) != exact_bits(y, dtype)
            assert not bad.any(), f"{tag}, problem {z}: {int(bad.sum())} outputs differ"


def test_strided_batch_weights_residual_and_drelu():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype, batch = 136, 208, 264, "fp16", 4  # each mask (m*n/8 bytes) 16-byte aligned
    a = W.normal_bits((m, k), 1.0, dtype, 7, 0)
    b_list = [W.normal_bits((k, n), 1.0 / np.sqrt(k) / 2, dtype, 8, z) for z in range(batch)]
    r_list = [W.normal_bits((m, n), 0.5, dtype, 9, z) for z in range(batch)]
    bias = W.normal_bits((m,), 0.5, dtype, 10, 0)
    # B batched, A shared; the residual advances with D
    with egm.Matmul(to_device(a, dtype), to_device(b_list[0], dtype)) as mm:
        mm.plan("BIAS_RESIDUAL", {"bias": bias_tensor(bias, "row", dtype), "residual": _stack(r_list, dtype)})
        d = mm.execute_batched(to_device(a, dtype), _stack(b_list, dtype))
        torch.cuda.synchronize()
    for z in range(batch):
        y, _, _ = eo.reference(a, b_list[z], dtype, "BIAS_RESIDUAL", bias, "row", r_list[z])
        compare(to_host_bits(d[z]), y, dtype)
    # a residual of one problem cannot serve a batch (it advances with D)
    with egm.Matmul(to_device(a, dtype), to_device(b_list[0], dtype)) as mm:
        mm.plan("BIAS_RESIDUAL", {"bias": bias_tensor(bias, "row", dtype), "residual": to_device(r_list[0], dtype)})
        with pytest.raises(ValueError):
            mm.execute_batched(to_device(a, dtype), _stack(b_list, dtype))
    # DRELU: one input mask per problem
    masks = [np.random.default_rng(z).integers(0, 256, size=(m, n // 8), dtype=np.uint8) for z in range(batch)]
    aux = torch.from_numpy(np.stack(masks)).cuda()
    with egm.Matmul(to_device(a, dtype), to_device(b_list[0], dtype)) as mm:
        mm.plan("DRELU")
        d = mm.execute_batched(to_device(a, dtype), _stack(b_list, dtype), aux=aux)
        torch.cuda.synchronize()
    for z in range(batch):
        dz, _, _ = eo.backward_reference(a, b_list[z], dtype, "DRELU", masks[z])
        compare(to_host_bits(d[z]), dz, dtype)


def test_strided_batch_fp8():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, batch = 200, 144, 320, 3
    probs = [W.fp8_operands(m, n, k, "e4m3", "e5m2", "bf16", seed=70 + z, b_std=0.4 / np.sqrt(k), bias_layout="col",
                            bias_std=0.3) for z in range(batch)]
    # one scale pair for the whole launch: requantise every problem with problem 0's scales
    sa, sb = probs[0].scale_a, probs[0].scale_b
    a_list = [W.f32_to_fp8_bits(eo.decode_fp8(p.a, "e4m3").astype(np.float32) * p.scale_a / sa, "e4m3") for p in probs]
    b_list = [W.f32_to_fp8_bits(eo.decode_fp8(p.b, "e5m2").astype(np.float32) * p.scale_b / sb, "e5m2") for p in probs]
    a_dev = torch.stack([fp8_to_device(x, "e4m3") for x in a_list])
    b_dev = torch.stack([fp8_to_device(x, "e5m2") for x in b_list])
    with egm.Matmul(a_dev[0], b_dev[0], scale_a=scale_tensor(sa), scale_b=scale_tensor(sb),
                    out_dtype=torch.bfloat16) as mm:
        mm.plan("GELU_BIAS", {"bias": bias_tensor(probs[0].bias, "col", "bf16")})
        d = mm.execute_batched(a_dev, b_dev)
        torch.cuda.synchronize()
    for z in range(batch):
        y, _, _ = eo.reference_fp8(a_list[z], b_list[z], "e4m3", "e5m2", sa, sb, "bf16", "GELU_BIAS", probs[0].bias,
                                   "col")
        compare(to_host_bits(d[z]), y, "bf16")


def test_graph_capture_replays_match_eager():
    """Executes of several plans (fused forward, the two-kernel path, the
    two-launch bias gradient, fp8, a strided batch) captured in one HIP graph;
    each of three replays, separated by eager work that overwrites the outputs
    and a synchronize, reproduces the eager results exactly."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k = 264, 208, 144  # n, k multiples of 16 for the fp8 plan
    ops = W.gemm_operands(m, n, k, "bf16", seed=3, a_std=1.0, b_std=1.0 / np.sqrt(k), bias_layout="col",
                          bias_std=0.5, residual_std=0.5)
    a, b = to_device(ops.a, "bf16"), to_device(ops.b, "bf16")
    bias = bias_tensor(ops.bias, "col", "bf16")
    grad = torch.empty((1, n), dtype=torch.float32, device="cuda")
    f8 = W.fp8_operands(m, n, k, "e4m3", "e4m3", "bf16", seed=4, bias_layout="col")
    a8, b8 = fp8_to_device(f8.a, "e4m3"), fp8_to_device(f8.b, "e4m3")
    mm_aux, mm_unf, mm_bg = egm.Matmul(a, b), egm.Matmul(a, b), egm.Matmul(a, b)
    mm_f8 = egm.Matmul(a8, b8, scale_a=scale_tensor(f8.scale_a), scale_b=scale_tensor(f8.scale_b),
                       out_dtype=torch.bfloat16)
    mm_b = egm.Matmul(a, b)
    mm_aux.plan("RELU_AUX_BIAS", {"bias": bias})
    mm_unf.plan("GELU_BIAS", {"bias": bias}, fused=False)
    mm_bg.plan("DRELU_BGRAD", {"bias_grad": grad})
    mm_f8.plan("RELU_BIAS", {"bias": bias_tensor(f8.bias, "col", "bf16")})
    mm_b.plan("BIAS", {"bias": bias})
    outs = {name: torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for name in ("aux", "unf", "bg", "f8")}
    mask = torch.empty((m, n // 8), dtype=torch.uint8, device="cuda")
    a_batch = torch.stack([a, a * 0.5, -a])
    d_batch = torch.empty((3, m, n), dtype=torch.bfloat16, device="cuda")

    def work():
        mm_aux.execute(out=outs["aux"], aux=mask)
        mm_unf.execute(out=outs["unf"])
        mm_bg.execute(out=outs["bg"], aux=mask)  # consumes the mask written just before
        mm_f8.execute(out=outs["f8"])
        mm_b.execute_batched(a_batch, b, out=d_batch)

    work()
    torch.cuda.synchronize()
    want = {kk: v.clone() for kk, v in outs.items()}
    want_mask, want_grad, want_batch = mask.clone(), grad.clone(), d_batch.clone()
    # sanity against the oracle for the forward mask pass
    y, z, mref = eo.reference(ops.a, ops.b, "bf16", "RELU_AUX_BIAS", ops.bias, "col")
    compare(to_host_bits(want["aux"]), y, "bf16", z=z, mask=want_mask.cpu().numpy(), mask_ref=mref)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()  # a warm-up on the capture stream, outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for v in list(outs.values()) + [d_batch]:
            v.fill_(float("nan"))  # eager work between replays
        mask.fill_(0)
        grad.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kk in outs:
            assert torch.equal(outs[kk].view(torch.int16), want[kk].view(torch.int16)), (rep, kk)
        assert torch.equal(mask, want_mask) and torch.equal(grad, want_grad), rep
        assert torch.equal(d_batch.view(torch.int16), want_batch.view(torch.int16)), rep
    for mm in (mm_aux, mm_unf, mm_bg, mm_f8, mm_b):
        mm.free()


def test_binding_rejects_bad_output_buffers():
    """Wrong-sized, wrong-typed or strided outputs are refused on the host:
    the library cannot see buffer sizes, so a short buffer would be written
    past its end."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    a = torch.zeros((64, 32), dtype=torch.float16, device="cuda")
    b = torch.zeros((32, 48), dtype=torch.float16, device="cuda")
    bias = torch.zeros((1, 48), dtype=torch.float16, device="cuda")
    with egm.Matmul(a, b) as mm:
        mm.plan("RELU_AUX_BIAS", {"bias": bias})
        for bad in (torch.empty((64, 40), dtype=torch.float16, device="cuda"),
                    torch.empty((64, 48), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((48, 64), dtype=torch.float16, device="cuda").t()):
            with pytest.raises(ValueError):
                mm.execute(out=bad)
        with pytest.raises(ValueError):
            mm.execute(aux=torch.empty((64, 5), dtype=torch.uint8, device="cuda"))
        with pytest.raises(ValueError):
            mm.execute_batched(torch.zeros((2, 64, 32), dtype=torch.float16, device="cuda"), b,
                               out=torch.empty((1, 64, 48), dtype=torch.float16, device="cuda"))
        d, m = mm.execute()
        torch.cuda.synchronize()
        assert d.shape == (64, 48) and m.shape == (64, 6)
    with egm.Matmul(a, b) as mm:
        mm.plan("BIAS", {"bias": bias})
        with pytest.raises(ValueError):
            mm.execute(aux=torch.empty((64, 6), dtype=torch.uint8, device="cuda"))
