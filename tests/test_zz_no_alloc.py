"""egm_execute_no_alloc on the GPU, through the C ABI: the entry point for
callers that cannot allocate device memory takes its workspace from the
library's static per-GPU scratch.  Its outputs must equal egm_execute's (the
same kernels on the same inputs, bit for bit) and the CPU oracle's (to the
parity bar), on two calls in a row, the second with a smaller problem that
reuses the scratch the first left behind; and replays of a HIP graph that
captured it must reproduce the eager results."""
import numpy as np
import pytest

import egm_workloads as W
from oracle import egm_oracle as eo
from parity import bias_tensor, compare, compare_bias_grad, to_device, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_epilogue_fp16_amd  # noqa: F401  (fails loudly without libegm.so)


def _raw_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _bgrad_case(m, n, k, layout, seed):
    """DRELU_BGRAD (per-tile partial sums in the scratch): egm_execute with a
    caller workspace vs egm_execute_no_alloc, then the oracle."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    dtype = "bf16"
    print(f"[no-alloc DRELU_BGRAD {m}x{n}x{k} {layout}]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=seed, a_std=1.0, b_std=1.0 / np.sqrt(k), bias_layout=layout)
    mask = np.random.default_rng(seed + 1).integers(0, 256, size=(m, n // 8), dtype=np.uint8)
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    aux = torch.from_numpy(mask).cuda()
    shape = (m, 1) if layout == "row" else (1, n)
    g_ref_dev = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    g_na = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    d_ref = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    lay = egm.EGM_BIAS_ROW if layout == "row" else egm.EGM_BIAS_COL
    p_ref = egm.egm_plan(m, n, k, egm.EGM_BF16, egm.EPILOGS["DRELU_BGRAD"], 0, lay, bias_grad=g_ref_dev.data_ptr())
    p_na = egm.egm_plan(m, n, k, egm.EGM_BF16, egm.EPILOGS["DRELU_BGRAD"], 0, lay, bias_grad=g_na.data_ptr())
    try:
        wsb = egm.egm_plan_workspace_bytes(p_ref)
        assert 0 < wsb <= egm.EGM_NO_ALLOC_SCRATCH_BYTES
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        egm.egm_execute(p_ref, a.data_ptr(), b.data_ptr(), d_ref.data_ptr(), aux.data_ptr(), ws.data_ptr(), wsb,
                        _raw_stream())
        egm.egm_execute_no_alloc(p_na, a.data_ptr(), b.data_ptr(), d_na.data_ptr(), aux.data_ptr(), _raw_stream())
        torch.cuda.synchronize()
    finally:
        egm.egm_free(p_ref)
        egm.egm_free(p_na)
    assert torch.equal(d_na.view(torch.int16), d_ref.view(torch.int16))
    assert torch.equal(g_na, g_ref_dev)
    dz, g_want, bound = eo.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, layout)
    st = compare(to_host_bits(d_na), dz, dtype)
    gs = compare_bias_grad(g_na.double().cpu().numpy().reshape(-1), g_want, bound)
    print(f"  D {st} grad {gs}", flush=True)


def _unfused_case(m, n, k, epilog, dtype, layout, seed):
    """The two-kernel path (the intermediate product in the scratch)."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    print(f"[no-alloc unfused {epilog} {m}x{n}x{k} {dtype} {layout}]", flush=True)
    ops = W.gemm_operands(m, n, k, dtype, seed=seed, a_std=1.0, b_std=1.0 / np.sqrt(k) / 2, bias_layout=layout,
                          bias_std=0.5)
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    bias = bias_tensor(ops.bias, layout, dtype)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    d_ref = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
    d_na = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
    mask_ref = mask_na = None
    if epilog == "RELU_AUX_BIAS":
        mask_ref = torch.zeros((m, n // 8), dtype=torch.uint8, device="cuda")
        mask_na = torch.full((m, n // 8), 0x5A, dtype=torch.uint8, device="cuda")
    code = egm.EGM_F16 if dtype == "fp16" else egm.EGM_BF16
    lay = egm.EGM_BIAS_ROW if layout == "row" else egm.EGM_BIAS_COL
    p = egm.egm_plan(m, n, k, code, egm.EPILOGS[epilog], bias.data_ptr(), lay, fused=0)
    try:
        wsb = egm.egm_plan_workspace_bytes(p)
        assert 0 < wsb <= egm.EGM_NO_ALLOC_SCRATCH_BYTES
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        egm.egm_execute(p, a.data_ptr(), b.data_ptr(), d_ref.data_ptr(),
                        mask_ref.data_ptr() if mask_ref is not None else 0, ws.data_ptr(), wsb, _raw_stream())
        egm.egm_execute_no_alloc(p, a.data_ptr(), b.data_ptr(), d_na.data_ptr(),
                                 mask_na.data_ptr() if mask_na is not None else 0, _raw_stream())
        torch.cuda.synchronize()
    finally:
        egm.egm_free(p)
    assert torch.equal(d_na.view(torch.int16), d_ref.view(torch.int16))
    if mask_na is not None:
        assert torch.equal(mask_na, mask_ref)
    y, z, mref = eo.reference(ops.a, ops.b, dtype, epilog, ops.bias, layout)
    st = compare(to_host_bits(d_na), y, dtype, z=z, mask=None if mask_na is None else mask_na.cpu().numpy(),
                 mask_ref=mref, unfused=True)
    print(f"  {st}", flush=True)


def test_two_calls_in_a_row_second_smaller():
    """Largest first, then a smaller problem on the scratch the first left:
    the bias gradient's partials (about 1.3 MiB, then 0.3 MiB), and the
    two-kernel path's product (about 1 MiB, then 70 KiB)."""
    _bgrad_case(1000, 1040, 264, "col", seed=81)
    _bgrad_case(300, 264, 136, "row", seed=82)
    _unfused_case(1024, 512, 2048, "RELU_AUX_BIAS", "fp16", "row", seed=83)
    _unfused_case(264, 136, 72, "GELU_BIAS", "bf16", "col", seed=84)


def test_fused_plan_needs_no_scratch():
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype = 520, 392, 328, "fp16"
    ops = W.gemm_operands(m, n, k, dtype, seed=85, bias_layout="row")
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    bias = bias_tensor(ops.bias, "row", dtype)
    d = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    p = egm.egm_plan(m, n, k, egm.EGM_F16, egm.EPILOGS["RELU_BIAS"], bias.data_ptr(), egm.EGM_BIAS_ROW)
    try:
        assert egm.egm_plan_workspace_bytes(p) == 0
        egm.egm_execute_no_alloc(p, a.data_ptr(), b.data_ptr(), d.data_ptr(), 0, _raw_stream())
        torch.cuda.synchronize()
    finally:
        egm.egm_free(p)
    y, _, _ = eo.reference(ops.a, ops.b, dtype, "RELU_BIAS", ops.bias, "row")
    print("[no-alloc fused RELU_BIAS]", compare(to_host_bits(d), y, dtype), flush=True)


def test_refusals_enqueue_nothing():
    """A plan needing more than the static scratch, and a pending autotune,
    are refused on the host; D keeps its poison."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k = 4096, 8192, 64  # the two-kernel product alone is 64 MiB
    a = torch.zeros((m, k), dtype=torch.float16, device="cuda")
    b = torch.zeros((k, n), dtype=torch.float16, device="cuda")
    bias = torch.zeros((m, 1), dtype=torch.float16, device="cuda")
    d = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    p = egm.egm_plan(m, n, k, egm.EGM_F16, egm.EPILOGS["BIAS"], bias.data_ptr(), egm.EGM_BIAS_ROW, fused=0)
    q = egm.egm_plan(256, 256, 64, egm.EGM_F16, egm.EPILOGS["BIAS"], bias.data_ptr(), egm.EGM_BIAS_ROW, fused=0,
                     autotune=1)
    try:
        assert egm.egm_plan_workspace_bytes(p) > egm.EGM_NO_ALLOC_SCRATCH_BYTES
        st = egm.egm_execute_no_alloc(p, a.data_ptr(), b.data_ptr(), d.data_ptr(), 0, _raw_stream(), raw_status=True)
        assert st == egm.EGM_ERR_SCRATCH_LIMIT, egm.status_string(st)
        st = egm.egm_execute_no_alloc(q, a.data_ptr(), b.data_ptr(), d.data_ptr(), 0, _raw_stream(), raw_status=True)
        assert st == egm.EGM_ERR_NOT_SUPPORTED, egm.status_string(st)
        torch.cuda.synchronize()
        assert torch.isnan(d).all()
    finally:
        egm.egm_free(p)
        egm.egm_free(q)


def test_graph_capture_replays():
    """Captured in a HIP graph (the callers this entry point is for): the
    two-kernel path and the bias gradient, replayed three times with eager
    writes between the replays, each replay equal to the eager result."""
    import torch
    import dense_gemm_epilogue_fp16_amd as egm
    m, n, k, dtype = 264, 208, 144, "bf16"
    ops = W.gemm_operands(m, n, k, dtype, seed=86, a_std=1.0, b_std=1.0 / np.sqrt(k), bias_layout="col",
                          bias_std=0.5)
    a, b = to_device(ops.a, dtype), to_device(ops.b, dtype)
    bias = bias_tensor(ops.bias, "col", dtype)
    mask = torch.from_numpy(np.random.default_rng(87).integers(0, 256, size=(m, n // 8), dtype=np.uint8)).cuda()
    grad = torch.empty((1, n), dtype=torch.float32, device="cuda")
    d_unf = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    d_bg = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    p_unf = egm.egm_plan(m, n, k, egm.EGM_BF16, egm.EPILOGS["GELU_BIAS"], bias.data_ptr(), egm.EGM_BIAS_COL, fused=0)
    p_bg = egm.egm_plan(m, n, k, egm.EGM_BF16, egm.EPILOGS["DRELU_BGRAD"], 0, egm.EGM_BIAS_COL,
                        bias_grad=grad.data_ptr())

    def work():
        s = _raw_stream()
        egm.egm_execute_no_alloc(p_unf, a.data_ptr(), b.data_ptr(), d_unf.data_ptr(), 0, s)
        egm.egm_execute_no_alloc(p_bg, a.data_ptr(), b.data_ptr(), d_bg.data_ptr(), mask.data_ptr(), s)

    try:
        work()
        torch.cuda.synchronize()
        want_unf, want_bg, want_grad = d_unf.clone(), d_bg.clone(), grad.clone()
        y, _, _ = eo.reference(ops.a, ops.b, dtype, "GELU_BIAS", ops.bias, "col")
        compare(to_host_bits(want_unf), y, dtype, unfused=True)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            work()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            work()
        for rep in range(3):
            d_unf.fill_(float("nan"))
            d_bg.fill_(float("nan"))
            grad.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(d_unf.view(torch.int16), want_unf.view(torch.int16)), rep
            assert torch.equal(d_bg.view(torch.int16), want_bg.view(torch.int16)), rep
            assert torch.equal(grad, want_grad), rep
    finally:
        egm.egm_free(p_unf)
        egm.egm_free(p_bg)
