"""C-ABI library: loads, exports every declared symbol, validates arguments on
the host before any HIP call (CPU only: no test here launches a kernel)."""
import ctypes
import os
import re

import pytest

import dense_gemm_epilogue_fp16_amd as egm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "egm.h")

F16, BF16 = egm.EGM_F16, egm.EGM_BF16
E = egm.EPILOGS
ROW, COL = egm.EGM_BIAS_ROW, egm.EGM_BIAS_COL
FAKE = 0x7F0000000000  # a 256-byte aligned address; never dereferenced by plan()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:egm_status_t|size_t|int32_t|const char\*)\s+(egm_\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 14
    assert sorted(egm.EXPORTS) == names
    lib = ctypes.CDLL(egm.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert egm.egm_abi_version() == 7
    for s in range(11):
        assert egm.status_string(s).startswith("EGM_")
    assert "unknown" in egm.status_string(12345)


def plan_status(m=64, n=64, k=64, dtype=F16, epilog="BIAS", bias=FAKE, layout=ROW, residual=0, **kw):
    st, h = egm.egm_plan(m, n, k, dtype, E[epilog] if isinstance(epilog, str) else epilog, bias, layout,
                         residual, raw_status=True, **kw)
    if h:
        assert egm.egm_free(h, raw_status=True) == egm.EGM_OK
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(), egm.EGM_OK),
    (dict(m=-1), egm.EGM_ERR_SHAPE),
    (dict(n=12), egm.EGM_ERR_SHAPE),
    (dict(k=20), egm.EGM_ERR_SHAPE),
    (dict(n=(1 << 21) + 8), egm.EGM_ERR_SHAPE),
    (dict(k=(1 << 21) + 8), egm.EGM_ERR_SHAPE),
    (dict(n=1 << 21, k=1 << 21), egm.EGM_OK),
    (dict(m=1 << 31), egm.EGM_ERR_SHAPE),
    (dict(dtype=2), egm.EGM_ERR_DTYPE),
    (dict(epilog=8), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="DRELU", bias=0, layout=0), egm.EGM_OK),
    (dict(epilog="DRELU"), egm.EGM_ERR_INVALID_VALUE),            # no bias in the backward epilogues
    (dict(epilog="DRELU", bias=0, layout=0, bias_grad=FAKE), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="DRELU_BGRAD", bias=0, bias_grad=FAKE), egm.EGM_OK),
    (dict(epilog="DRELU_BGRAD", bias=0, layout=COL, bias_grad=FAKE), egm.EGM_OK),
    (dict(epilog="DRELU_BGRAD", bias=0, bias_grad=0), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="DRELU_BGRAD", bias=0, layout=0, bias_grad=FAKE), egm.EGM_ERR_SHAPE),
    (dict(epilog="DRELU_BGRAD", bias=0, bias_grad=FAKE + 4), egm.EGM_ERR_ALIGNMENT),
    (dict(epilog="DRELU_BGRAD", bias_grad=FAKE), egm.EGM_ERR_INVALID_VALUE),   # a bias as well
    (dict(epilog="BIAS", bias_grad=FAKE), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog=-1), egm.EGM_ERR_INVALID_VALUE),
    (dict(bias=0), egm.EGM_ERR_INVALID_VALUE),
    (dict(layout=0), egm.EGM_ERR_SHAPE),
    (dict(layout=3), egm.EGM_ERR_SHAPE),
    (dict(bias=FAKE + 8), egm.EGM_ERR_ALIGNMENT),
    (dict(epilog="BIAS_RESIDUAL"), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="BIAS_RESIDUAL", residual=FAKE + 2), egm.EGM_ERR_ALIGNMENT),
    (dict(epilog="BIAS_RESIDUAL", residual=FAKE + 4096), egm.EGM_OK),
    (dict(epilog="RELU_BIAS", residual=FAKE + 4096), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="DEFAULT"), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="DEFAULT", bias=0, layout=0), egm.EGM_OK),
    (dict(m=0), egm.EGM_OK),
    (dict(n=0), egm.EGM_OK),
    (dict(k=0), egm.EGM_OK),
    (dict(fused=2), egm.EGM_ERR_INVALID_VALUE),
    (dict(force_config=99), egm.EGM_ERR_INVALID_VALUE),
    (dict(force_config=-2), egm.EGM_ERR_INVALID_VALUE),
    (dict(autotune=1, force_config=0), egm.EGM_ERR_INVALID_VALUE),
    (dict(autotune=1), egm.EGM_OK),
    (dict(group_m=-1), egm.EGM_ERR_INVALID_VALUE),
    (dict(epilog="GELU_BIAS", dtype=BF16, layout=COL), egm.EGM_OK),
    (dict(epilog="RELU_AUX_BIAS", dtype=BF16, layout=COL, n=8), egm.EGM_OK),
])
def test_plan_validation(kw, status):
    assert plan_status(**kw) == status


def test_plan_null_out_pointer():
    ins = egm.EpilogInputs(FAKE, ROW, None)
    assert egm.LIB.egm_plan(None, 8, 8, 8, F16, E["BIAS"], ctypes.byref(ins), None) == egm.EGM_ERR_INVALID_VALUE
    h = ctypes.c_void_p(123)
    # NULL options are the defaults
    assert egm.LIB.egm_plan(ctypes.byref(h), 8, 8, 8, F16, E["BIAS"], ctypes.byref(ins), None) == egm.EGM_OK
    assert h.value
    assert egm.egm_plan_config(h.value) >= 0
    egm.egm_free(h.value)


def test_free_and_invalid_handles():
    assert egm.egm_free(0, raw_status=True) == egm.EGM_OK
    assert egm.egm_execute(0, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    assert egm.egm_plan_workspace_bytes(0) == 0
    assert egm.egm_plan_config(0) == -1
    assert egm.LIB.egm_plan_describe(None, ctypes.create_string_buffer(8), 8) == egm.EGM_ERR_INVALID_PLAN


def test_freed_handles_are_rejected_and_never_reused():
    """A freed handle is refused by every call (double free included) without
    the library touching the freed plan; a later plan gets a new handle."""
    h = egm.egm_plan(64, 64, 64, F16, E["BIAS"], FAKE, ROW)
    assert egm.egm_free(h, raw_status=True) == egm.EGM_OK
    assert egm.egm_free(h, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    assert egm.egm_execute(h, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    assert egm.egm_execute_strided(h, 1, FAKE, 0, FAKE, 0, FAKE, 0, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    assert egm.egm_plan_workspace_bytes(h) == 0
    assert egm.egm_plan_config(h) == -1
    assert egm.LIB.egm_plan_describe(h, ctypes.create_string_buffer(64), 64) == egm.EGM_ERR_INVALID_PLAN
    seen = {h}
    for _ in range(64):
        h2 = egm.egm_plan(64, 64, 64, F16, E["BIAS"], FAKE, ROW)
        assert h2 not in seen
        seen.add(h2)
        assert egm.egm_free(h2, raw_status=True) == egm.EGM_OK
    # a foreign value that was never a handle
    for bogus in (1, 0x1008, FAKE):
        assert egm.egm_free(bogus, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
        assert egm.egm_plan_config(bogus) == -1


def test_out_of_range_enum_values_are_rejected():
    """Any int32 may arrive where an enum is expected; unknown ones give a status."""
    for dt in (2, -1, 1 << 30):
        assert plan_status(dtype=dt) == egm.EGM_ERR_DTYPE
    for ep in (8, -7, 1 << 30):
        assert plan_status(epilog=ep) == egm.EGM_ERR_INVALID_VALUE
    for st in (11, -1, (1 << 31) - 1):
        assert "unknown" in egm.status_string(st)


def test_workspace_and_describe():
    h = egm.egm_plan(256, 512, 64, F16, E["RELU_BIAS"], FAKE, ROW, fused=0)
    try:
        assert egm.egm_plan_workspace_bytes(h) == 256 * 512 * 2
        d = egm.egm_plan_describe(h)
        assert "unfused" in d and "RELU_BIAS" in d and "row(m,1)" in d
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(256, 512, 64, F16, E["RELU_BIAS"], FAKE, ROW)
    try:
        assert egm.egm_plan_workspace_bytes(h) == 0
        assert "path=fused" in egm.egm_plan_describe(h)
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(256, 512, 64, F16, E["DEFAULT"], fused=0)
    try:
        assert egm.egm_plan_workspace_bytes(h) == 0  # nothing to keep apart for a bare product
    finally:
        egm.egm_free(h)


def test_execute_validation_before_any_hip_call(monkeypatch):
    h = egm.egm_plan(64, 64, 64, F16, E["RELU_AUX_BIAS"], FAKE, COL)
    try:
        # the mask is required for RELU_AUX_BIAS
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
        assert egm.egm_execute(h, FAKE, FAKE, 0, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
        assert egm.egm_execute(h, FAKE + 2, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_ALIGNMENT
        assert egm.egm_execute(h, FAKE, FAKE + 8, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_ALIGNMENT
        assert egm.egm_execute(h, FAKE, FAKE, FAKE + 4, FAKE, raw_status=True) == egm.EGM_ERR_ALIGNMENT
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, FAKE + 1, raw_status=True) == egm.EGM_ERR_ALIGNMENT
        assert egm.egm_execute(h, 0, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
        monkeypatch.setenv("EGM_FAIL_INJECT", "launch")
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_HIP
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(64, 64, 64, F16, E["BIAS"], FAKE, ROW)
    try:
        # a mask for an epilog that has none
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(64, 64, 64, F16, E["BIAS"], FAKE, ROW, fused=0)
    try:
        need = egm.egm_plan_workspace_bytes(h)
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, 0, 0, raw_status=True) == egm.EGM_ERR_WORKSPACE
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, FAKE, need - 1, raw_status=True) == egm.EGM_ERR_WORKSPACE
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, FAKE + 8, need, raw_status=True) == egm.EGM_ERR_ALIGNMENT
    finally:
        egm.egm_free(h)
    # empty output: nothing to launch, OK without touching the device
    h = egm.egm_plan(0, 64, 64, F16, E["BIAS"], FAKE, ROW)
    try:
        assert egm.egm_execute(h, 0, 0, 0, raw_status=True) == egm.EGM_OK
    finally:
        egm.egm_free(h)


@pytest.mark.parametrize("m,n,k,cfg", [
    (256, 256, 512, 6),       # small square: 32 tiles of 32x64 (16x16x32 blocks, 16-bit operands)
    (1024, 512, 2048, 6),     # the bias-fusion page's example shape: 256 tiles of 32x64, one per CU
    (4096, 4096, 1024, 0),    # FFN up-projection: 256 tiles of 256x256, one per CU (K below 2048)
    (4096, 4096, 2040, 0),
    (4096, 4096, 2048, 7),    # from K = 2048 on: the lean 256x256 tile (16x16x32 blocks)
    (4096, 1024, 4096, 3),    # FFN down-projection: 256 tiles of 128x128
    (8192, 8192, 8192, 7),
    (65536, 16384, 16384, 7),
])
def test_per_shape_choice(m, n, k, cfg):
    # a forward epilogue without the mask, B not transposed
    h = egm.egm_plan(m, n, k, F16, E["BIAS"], FAKE, ROW)
    try:
        assert egm.egm_plan_config(h) == cfg
    finally:
        egm.egm_free(h)


@pytest.mark.parametrize("kind", ["mask", "b_transposed", "backward"])
@pytest.mark.parametrize("k,cfg", [(8192, 0), (12280, 0), (12288, 7), (16384, 7)])
def test_per_shape_choice_long_k_only(kind, k, cfg):
    # the mask epilogue, B transposed and the backward epilogues take the lean
    # tile only from K = 12288 on
    kw = dict(epilog=E["BIAS"], bias=FAKE, bias_layout=ROW)
    if kind == "mask":
        kw["epilog"] = E["RELU_AUX_BIAS"]
    elif kind == "b_transposed":
        kw["b_transposed"] = 1
    else:
        kw = dict(epilog=E["DRELU_BGRAD"], bias=0, bias_layout=ROW, bias_grad=FAKE)
    h = egm.egm_plan(8192, 8192, k, F16, kw.pop("epilog"), kw.pop("bias"), kw.pop("bias_layout"), **kw)
    try:
        assert egm.egm_plan_config(h) == cfg
    finally:
        egm.egm_free(h)


@pytest.mark.parametrize("epilog", ["DEFAULT", "BIAS", "RELU_AUX_BIAS", "DRELU"])
@pytest.mark.parametrize("fused,cfg", [(1, None), (0, 7)])
def test_per_shape_choice_two_kernel_path(epilog, fused, cfg):
    # on the two-kernel path the GEMM kernel applies no epilogue (a second
    # kernel does), so its GEMM takes the lean tile at K = 8192 whatever the
    # epilogue; fused, only the epilogues without the mask do
    if cfg is None:
        cfg = 0 if epilog in ("RELU_AUX_BIAS", "DRELU") else 7
    bias, layout = (FAKE, ROW) if epilog in ("BIAS", "RELU_AUX_BIAS") else (0, egm.EGM_BIAS_NONE)
    h = egm.egm_plan(8192, 8192, 8192, F16, E[epilog], bias, layout, fused=fused)
    try:
        assert egm.egm_plan_config(h) == cfg
    finally:
        egm.egm_free(h)


def test_fp8_long_k_keeps_the_32x32_tile():
    # the lean tile has 16x16x32 blocks, which exist for 16-bit operands only
    h = egm.egm_plan_fp8(8192, 8192, 16384, egm.EGM_E4M3, egm.EGM_E4M3, BF16, FAKE, FAKE, E["BIAS"], FAKE, COL)
    try:
        assert egm.egm_plan_config(h) == 0
    finally:
        egm.egm_free(h)


def grid_work_items(m, n, cfg):
    d = dict(kv.split("=") for kv in egm.egm_config_describe(cfg).split())
    bm, bn = (int(x) for x in d["tile"].split("x"))
    wm, wn = (int(x) for x in d["waves"].split("x"))
    return -(-m // bm) * -(-n // bn) * 64 * wm * wn


def test_grid_limit_narrows_the_choice():
    # one workgroup per tile in one grid dimension, at most 2^32 - 1
    # work-items: for m = 2^31 - 1, n = 8 only the 256-row tiles of 4 waves
    # fit; every 128- or 64-row tile and the 8-wave 256x256 tile would not
    m = (1 << 31) - 1
    fits = [c for c in range(egm.egm_num_configs()) if grid_work_items(m, 8, c) <= 0xFFFFFFFF]
    described = [dict(kv.split("=") for kv in egm.egm_config_describe(c).split()) for c in fits]
    assert 1 in fits and all(d["tile"].startswith("256x") and d["waves"] == "2x2" for d in described)
    for kw in (dict(), dict(autotune=1)):
        h = egm.egm_plan(m, 8, 8, F16, E["BIAS"], FAKE, ROW, **kw)
        try:
            assert egm.egm_plan_config(h) == 1
        finally:
            egm.egm_free(h)
    for c in range(egm.egm_num_configs()):
        assert plan_status(m=m, n=8, k=8, force_config=c) == (egm.EGM_OK if c in fits else egm.EGM_ERR_NOT_SUPPORTED)
    # just over 2^30 rows (the parity test's shape): the small tiles drop out
    m = (1 << 30) + 200
    h = egm.egm_plan(m, 8, 8, F16, E["BIAS"], FAKE, ROW)
    try:
        c = egm.egm_plan_config(h)
        assert grid_work_items(m, 8, c) <= 0xFFFFFFFF
        assert grid_work_items(m, 8, 4) > 0xFFFFFFFF
    finally:
        egm.egm_free(h)
    # no config fits at all
    assert plan_status(m=(1 << 31) - 1, n=1 << 21, k=8) == egm.EGM_ERR_NOT_SUPPORTED
    # the workspace of a DRELU_BGRAD autotune plan covers only configs that fit
    st, h = egm.egm_plan((1 << 31) - 1, 8, 8, F16, E["DRELU_BGRAD"], 0, COL, bias_grad=FAKE, autotune=1,
                         raw_status=True)
    assert st == egm.EGM_OK
    try:
        assert egm.egm_plan_workspace_bytes(h) == -(-((1 << 31) - 1) // 256) * 8 * 4
    finally:
        egm.egm_free(h)


def test_config_table():
    n = egm.egm_num_configs()
    assert n == 8
    assert egm.egm_config_describe(0).startswith("tile=256x256 kslab=64 waves=2x4")
    d7 = egm.egm_config_describe(7)
    assert d7.startswith("tile=256x256 kslab=64 waves=2x4") and "mfma=16x16x32" in d7
    # configs of 16x16x32 MFMA blocks exist for 16-bit operands only
    for c in range(n):
        d = dict(kv.split("=") for kv in egm.egm_config_describe(c).split())
        st = egm.egm_plan_fp8(256, 256, 256, egm.EGM_E4M3, egm.EGM_E4M3, BF16, 0, 0, E["BIAS"], FAKE, COL,
                              force_config=c, raw_status=True)[0]
        if d["mfma"] == "16x16x32":
            assert d["operands"] == "16-bit" and st == egm.EGM_ERR_NOT_SUPPORTED
        else:
            assert d["mfma"] == "32x32x16" and st == egm.EGM_OK
    for c in range(n):
        d = dict(kv.split("=") for kv in egm.egm_config_describe(c).split())
        bm, bn = (int(x) for x in d["tile"].split("x"))
        wm, wn = (int(x) for x in d["waves"].split("x"))
        assert d["wave_tile"] == f"{bm // wm}x{bn // wn}"
        # the ring plus the tile's bias slice fit the 160 KiB of LDS
        assert int(d["lds_bytes"]) == int(d["lds_ring"]) * (bm + bn) * int(d["kslab"]) * 2
        assert int(d["lds_bytes"]) + 1024 <= 160 * 1024
    assert egm.LIB.egm_config_describe(n, ctypes.create_string_buffer(8), 8) == egm.EGM_ERR_INVALID_VALUE


def test_matmul_wrapper_rejects_without_gpu():
    import torch
    a = torch.zeros(8, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        egm.Matmul(a, a)  # CPU tensors are not device memory


def test_backward_workspace_and_execute_validation():
    # fused DRELU_BGRAD: fp32 partial sums, one row of n per tile row of a (1,n) bias
    h = egm.egm_plan(100, 64, 32, BF16, E["DRELU_BGRAD"], 0, COL, bias_grad=FAKE)
    try:
        bm = int(re.search(r"tile=(\d+)x(\d+)", egm.egm_plan_describe(h)).group(1))
        assert egm.egm_plan_workspace_bytes(h) == -(-100 // bm) * 64 * 4  # ceil(m/BM) rows x n x fp32
        assert "DRELU_BGRAD" in egm.egm_plan_describe(h)
        # the forward mask is an input here: required
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, FAKE, 4096, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, FAKE, 0, 0, raw_status=True) == egm.EGM_ERR_WORKSPACE
    finally:
        egm.egm_free(h)
    # autotuning may pick any tile: room for the shortest (32 rows: ceil(100/32) = 4 partial rows)
    h = egm.egm_plan(100, 64, 32, BF16, E["DRELU_BGRAD"], 0, COL, bias_grad=FAKE, autotune=1)
    try:
        assert egm.egm_plan_workspace_bytes(h) == 4 * 64 * 4
    finally:
        egm.egm_free(h)
    # (m,1) gradient, two-kernel path: one row of m per 32-column block of D, after P
    h = egm.egm_plan(100, 72, 32, F16, E["DRELU_BGRAD"], 0, ROW, bias_grad=FAKE, fused=0)
    try:
        p_bytes = (100 * 72 * 2 + 255) // 256 * 256
        assert egm.egm_plan_workspace_bytes(h) == p_bytes + 3 * 100 * 4  # ceil(72/32) = 3 blocks x m
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(64, 64, 64, F16, E["DRELU"], 0, 0)
    try:
        assert egm.egm_plan_workspace_bytes(h) == 0
        assert egm.egm_execute(h, FAKE, FAKE, FAKE, 0, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
    finally:
        egm.egm_free(h)


def test_fp8_plan_validation_and_describe():
    F8 = egm.EGM_E4M3, egm.EGM_E5M2
    E4, E5 = F8
    h = egm.egm_plan_fp8(256, 512, 1024, E4, E5, BF16, FAKE, FAKE + 4, E["RELU_AUX_BIAS"], FAKE, COL)
    try:
        d = egm.egm_plan_describe(h)
        assert "operands=e4m3xe5m2" in d and "dtype=bf16" in d and "mfma=32x32x64" in d and "kslab=128" in d
        assert egm.egm_plan_workspace_bytes(h) == 0
    finally:
        egm.egm_free(h)
    # NULL scales mean 1; every format pairing plans
    for fa in F8:
        for fb in F8:
            st, h = egm.egm_plan_fp8(64, 64, 64, fa, fb, F16, 0, 0, E["DEFAULT"], raw_status=True)
            assert st == egm.EGM_OK
            egm.egm_free(h)
    bad = [
        (dict(a_format=7), egm.EGM_ERR_DTYPE),
        (dict(b_format=-1), egm.EGM_ERR_DTYPE),
        (dict(out_dtype=5), egm.EGM_ERR_DTYPE),
        (dict(n=72), egm.EGM_ERR_SHAPE),   # a multiple of 8 but not of 16: half a 16-byte fp8 row
        (dict(k=24), egm.EGM_ERR_SHAPE),
        (dict(epilog=E["DRELU"]), egm.EGM_ERR_NOT_SUPPORTED),
        (dict(epilog=E["DRELU_BGRAD"]), egm.EGM_ERR_NOT_SUPPORTED),
        (dict(scale_a=FAKE + 2), egm.EGM_ERR_ALIGNMENT),
        (dict(scale_b=FAKE + 1), egm.EGM_ERR_ALIGNMENT),
        (dict(bias=FAKE + 8), egm.EGM_ERR_ALIGNMENT),
        (dict(bias=0), egm.EGM_ERR_INVALID_VALUE),
    ]
    for kw, want in bad:
        args = dict(m=64, n=64, k=64, a_format=E4, b_format=E4, out_dtype=BF16, scale_a=FAKE, scale_b=FAKE,
                    epilog=E["BIAS"], bias=FAKE, bias_layout=COL)
        args.update(kw)
        if args["epilog"] in (E["DRELU"], E["DRELU_BGRAD"]):
            args.update(bias=0, bias_layout=0)
        st, h = egm.egm_plan_fp8(args.pop("m"), args.pop("n"), args.pop("k"), args.pop("a_format"),
                                 args.pop("b_format"), args.pop("out_dtype"), args.pop("scale_a"),
                                 args.pop("scale_b"), args.pop("epilog"), args.pop("bias"),
                                 args.pop("bias_layout"), raw_status=True)
        assert st == want and h is None, (kw, st)


def test_execute_strided_validation_before_any_hip_call():
    h = egm.egm_plan(64, 64, 64, F16, E["RELU_AUX_BIAS"], FAKE, COL)
    try:
        def st(**kw):
            args = dict(batch=4, A=FAKE, stride_a=64 * 64, B=FAKE, stride_b=0, D=FAKE, stride_d=64 * 64, aux=FAKE,
                        stride_aux=64 * 8)
            args.update(kw)
            return egm.egm_execute_strided(h, args["batch"], args["A"], args["stride_a"], args["B"], args["stride_b"],
                                           args["D"], args["stride_d"], args["aux"], args["stride_aux"],
                                           raw_status=True)
        assert st(batch=-1) == egm.EGM_ERR_INVALID_VALUE
        assert st(batch=65536) == egm.EGM_ERR_INVALID_VALUE
        assert st(aux=0) == egm.EGM_ERR_INVALID_VALUE                # RELU_AUX_BIAS writes masks
        assert st(stride_d=64 * 64 - 8) == egm.EGM_ERR_INVALID_VALUE  # outputs would overlap
        assert st(stride_aux=64 * 8 - 16) == egm.EGM_ERR_INVALID_VALUE
        assert st(stride_a=-8) == egm.EGM_ERR_INVALID_VALUE
        assert st(stride_a=64 * 64 + 4) == egm.EGM_ERR_ALIGNMENT       # problem 1's A off 16 bytes
        assert st(stride_aux=64 * 8 + 8) == egm.EGM_ERR_ALIGNMENT
        assert st(D=0) == egm.EGM_ERR_INVALID_VALUE
        assert st(batch=0) == egm.EGM_OK                              # nothing to do, no HIP call
        assert egm.egm_execute_strided(0, 1, FAKE, 0, FAKE, 0, FAKE, 0, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    finally:
        egm.egm_free(h)
    # the two-kernel path and the bias gradient's per-launch partials do not batch
    h = egm.egm_plan(64, 64, 64, F16, E["BIAS"], FAKE, COL, fused=0)
    try:
        assert egm.egm_execute_strided(h, 2, FAKE, 4096, FAKE, 0, FAKE, 4096, raw_status=True) == \
            egm.EGM_ERR_NOT_SUPPORTED
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(64, 64, 64, F16, E["DRELU_BGRAD"], 0, COL, bias_grad=FAKE)
    try:
        assert egm.egm_execute_strided(h, 2, FAKE, 4096, FAKE, 0, FAKE, 4096, FAKE, 512, raw_status=True) == \
            egm.EGM_ERR_NOT_SUPPORTED
    finally:
        egm.egm_free(h)


def test_layernorm_validation_before_any_hip_call():
    def st(**kw):
        a = dict(rows=16, cols=1024, dtype=BF16, x=FAKE, residual=0, gamma=FAKE, beta=FAKE, eps=1e-5, y=FAKE, mean=0,
                 rstd=0)
        a.update(kw)
        return egm.egm_layernorm(a["rows"], a["cols"], a["dtype"], a["x"], a["residual"], a["gamma"], a["beta"],
                                 a["eps"], a["y"], a["mean"], a["rstd"], raw_status=True)
    assert st(cols=0) == egm.EGM_ERR_SHAPE
    assert st(cols=12) == egm.EGM_ERR_SHAPE          # not a multiple of 8
    assert st(cols=32768 + 8) == egm.EGM_ERR_SHAPE   # longer than one row kernel holds
    assert st(rows=-1) == egm.EGM_ERR_SHAPE
    assert st(dtype=9) == egm.EGM_ERR_DTYPE
    assert st(eps=-1.0) == egm.EGM_ERR_INVALID_VALUE
    assert st(eps=float("nan")) == egm.EGM_ERR_INVALID_VALUE
    assert st(x=0) == egm.EGM_ERR_INVALID_VALUE
    assert st(y=0) == egm.EGM_ERR_INVALID_VALUE
    assert st(gamma=FAKE + 2) == egm.EGM_ERR_ALIGNMENT
    assert st(residual=FAKE + 8) == egm.EGM_ERR_ALIGNMENT
    assert st(mean=FAKE + 2) == egm.EGM_ERR_ALIGNMENT
    assert st(rows=0) == egm.EGM_OK                  # nothing to do, no HIP call
    # one grid dimension of 256-thread workgroups (2^32 - 1 work-items): 4
    # rows per workgroup up to 4096 columns, 1 beyond
    assert st(rows=4 * ((1 << 24) - 1) + 1, cols=4096) == egm.EGM_ERR_NOT_SUPPORTED
    assert st(rows=(1 << 24), cols=4104) == egm.EGM_ERR_NOT_SUPPORTED


def test_b_transposed_option():
    h = egm.egm_plan(256, 512, 1024, BF16, E["BIAS"], FAKE, COL, b_transposed=1)
    try:
        assert " b=[n,k]" in egm.egm_plan_describe(h)
    finally:
        egm.egm_free(h)
    st, h = egm.egm_plan(256, 512, 1024, BF16, E["BIAS"], FAKE, COL, b_transposed=2, raw_status=True)
    assert st == egm.EGM_ERR_INVALID_VALUE and h is None
    st, h = egm.egm_plan_fp8(64, 64, 64, egm.EGM_E4M3, egm.EGM_E5M2, BF16, 0, 0, E["DEFAULT"], b_transposed=1,
                             raw_status=True)
    assert st == egm.EGM_OK
    egm.egm_free(h)


def test_execute_no_alloc_validation_before_any_hip_call():
    """The no-allocation entry point checks its arguments on the host first:
    handles, masks, pointers, the static scratch's size and a pending autotune
    (no GPU: none of these cases reaches a HIP call)."""
    assert egm.egm_execute_no_alloc(0, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_PLAN
    h = egm.egm_plan(4096, 8192, 64, F16, E["BIAS"], FAKE, ROW, fused=0)  # 64 MiB product
    try:
        assert egm.egm_plan_workspace_bytes(h) > egm.EGM_NO_ALLOC_SCRATCH_BYTES
        assert egm.egm_execute_no_alloc(h, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_SCRATCH_LIMIT
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(256, 256, 64, F16, E["BIAS"], FAKE, ROW, fused=0, autotune=1)
    try:
        assert egm.egm_execute_no_alloc(h, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_NOT_SUPPORTED
    finally:
        egm.egm_free(h)
    h = egm.egm_plan(256, 256, 64, F16, E["RELU_AUX_BIAS"], FAKE, ROW)
    try:
        assert egm.egm_execute_no_alloc(h, FAKE, FAKE, FAKE, 0, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
        assert egm.egm_execute_no_alloc(h, FAKE, FAKE, FAKE + 8, FAKE, raw_status=True) == egm.EGM_ERR_ALIGNMENT
        assert egm.egm_execute_no_alloc(h, FAKE, FAKE, 0, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_VALUE
    finally:
        egm.egm_free(h)
    assert egm.egm_execute_no_alloc(h, FAKE, FAKE, FAKE, FAKE, raw_status=True) == egm.EGM_ERR_INVALID_PLAN


def test_fp8_small_shapes_take_the_32x32_tile():
    """The 16x16x32 tile exists for 16-bit operands only: fp8 plans of the
    small shapes fall back to the 64x64 tile of 32x32x64 blocks."""
    for m, n, k in ((256, 256, 512), (1024, 512, 2048)):
        h = egm.egm_plan_fp8(m, n, k, egm.EGM_E4M3, egm.EGM_E4M3, BF16, 0, 0, E["BIAS"], FAKE, COL)
        try:
            assert egm.egm_plan_config(h) == 4
        finally:
            egm.egm_free(h)


def test_mfma_probe_library_exports_and_rejects():
    """The benchmark's MFMA-shape probe is a library of its own; its entry point
    refuses bad arguments before any HIP call (so this runs without a GPU)."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "dense_gemm_epilogue_fp16_amd", "libegm_probe.so")
    if not os.path.exists(path):
        pytest.skip("libegm_probe.so not built")
    lib = ctypes.CDLL(path)
    f = lib.egm_mfma_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(24, 10, 1, ctypes.c_void_p(16), None) == 1   # unknown shape
    assert f(32, 0, 1, ctypes.c_void_p(16), None) == 1    # no iterations
    assert f(16, 10, 0, ctypes.c_void_p(16), None) == 1   # no workgroups
    assert f(16, 10, 1, None, None) == 1                  # no output
