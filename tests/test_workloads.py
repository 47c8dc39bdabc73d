"""Seeded input generator: determinism, chunk recipe, operand rounding (CPU only)."""
import numpy as np
import pytest

import egm_workloads as W


def test_same_seed_same_bits_any_threads(monkeypatch):
    a = W.normal_bits((300, 50000), 0.1, W.BF16, seed=0, tensor_index=0)
    monkeypatch.setattr(W, "_THREADS", 1)
    b = W.normal_bits((300, 50000), 0.1, W.BF16, seed=0, tensor_index=0)
    assert np.array_equal(a, b)
    c = W.normal_bits((300, 50000), 0.1, W.BF16, seed=1, tensor_index=0)
    assert not np.array_equal(a, c)


def test_chunk_recipe():
    # the first chunk is exactly the documented stream, scaled in fp32, rounded once
    x = W.normal_bits((W.CHUNK + 5,), 0.25, W.F16, seed=3, tensor_index=2)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(3, spawn_key=(2, 0))))
    v = g.standard_normal(W.CHUNK, dtype=np.float32) * np.float32(0.25)
    assert np.array_equal(x[:W.CHUNK], v.astype(np.float16).view(np.uint16))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(3, spawn_key=(2, 1))))
    v = g.standard_normal(5, dtype=np.float32) * np.float32(0.25)
    assert np.array_equal(x[W.CHUNK:], v.astype(np.float16).view(np.uint16))


def test_bf16_operand_rounding_matches_torch():
    import torch
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * 3).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bits(x, W.BF16), want)
    assert np.array_equal(W.bits_to_f32(W.f32_to_bits(x, W.BF16), W.BF16),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_distribution_scale():
    x = W.bits_to_f32(W.normal_bits((1 << 20,), 1 / 64, W.BF16, 0, 0), W.BF16)
    assert abs(float(x.std()) - 1 / 64) < 1e-3 / 64 * 10
    assert abs(float(x.mean())) < 1e-4


def test_integer_operands_exact():
    ops = W.integer_operands(17, 24, 64, W.F16, seed=1, bias_layout="col", residual=True)
    for arr in (ops.a, ops.b, ops.bias, ops.residual):
        v = W.bits_to_f32(arr, W.F16)
        assert np.array_equal(v, np.round(v))
    assert ops.bias.shape == (24,)


def test_sample_rows():
    r = W.sample_rows(65536, 4096, seed=1)
    assert len(r) == 4096 and len(set(r.tolist())) == 4096
    assert r[0] == 0 and r[-1] == 65535 and np.all(np.diff(r) > 0)
    assert np.array_equal(r, W.sample_rows(65536, 4096, seed=1))
    assert np.array_equal(W.sample_rows(10, 20), np.arange(10))


def test_workload_table():
    names = list(W.WORKLOADS)
    assert len(names) == 5
    w = W.WORKLOADS["gemm_relu_bias_fp16_65536x16384x16384"]
    assert (w.m, w.n, w.k, w.dtype, w.bias_layout) == (65536, 16384, 16384, W.F16, "row")
    with pytest.raises(ValueError):
        W.workload_operands("ffn_bf16_4096x1024x4096")
    ops = W.workload_operands("gemm_bias_fp16_256x256x512")
    assert ops.a.shape == (256, 512) and ops.b.shape == (512, 256) and ops.bias.shape == (256,)


def test_backward_workload_and_mask_recipe():
    # the mask is uniform bytes from the same chunked streams (tensor index 2)
    m = W.mask_bits(64, 1024, seed=5, tensor_index=2)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(5, spawn_key=(2, 0))))
    assert m.shape == (64, 128) and m.dtype == np.uint8
    assert np.array_equal(m.reshape(-1), g.integers(0, 256, size=64 * 128, dtype=np.uint8))
    bits = np.unpackbits(W.mask_bits(512, 4096, seed=0, tensor_index=2))
    assert abs(float(bits.mean()) - 0.5) < 0.005  # ReLU-like density: half the pre-activations positive
    with pytest.raises(ValueError):
        W.mask_bits(4, 12, seed=0, tensor_index=2)
    w = W.BACKWARD_WORKLOADS["drelu_bgrad_bf16_8192x8192x8192"]
    assert (w.m, w.n, w.k, w.dtype, w.bias_layout) == (8192, 8192, 8192, W.BF16, "col")


def test_fp8_quantize_recipe():
    x = W.normal_f32((300, 70), 0.5, seed=4, tensor_index=0)
    assert np.array_equal(W.bits_to_f32(W.normal_bits((300, 70), 0.5, W.BF16, 4, 0), W.BF16),
                          W.bits_to_f32(W.f32_to_bits(x, W.BF16), W.BF16))  # the same draws
    for fmt in W.FP8:
        q, s = W.fp8_quantize(x, fmt)
        assert q.dtype == np.uint8 and q.shape == x.shape and s.dtype == np.float32
        assert s == np.float32(float(np.abs(x).max()) / W.FP8_MAX[fmt])
        import torch
        back = torch.from_numpy(q).view(torch.float8_e4m3fn if fmt == W.E4M3 else torch.float8_e5m2).float().numpy()
        assert np.abs(back).max() == W.FP8_MAX[fmt]  # amax maps to the largest finite value
        rel = np.abs(back * s - x) / np.maximum(np.abs(x), 1e-3)
        assert np.median(rel) < (2.0 ** -4 if fmt == W.E4M3 else 2.0 ** -3)
    # saturation instead of NaN beyond the largest finite value
    big = W.f32_to_fp8_bits(np.array([1e6, -1e6], dtype=np.float32), W.E4M3)
    assert list(big) == [0x7E, 0xFE]
    w = W.FP8_WORKLOADS["gemm_relu_aux_bias_fp8e4m3_8192x8192x8192"]
    assert (w.m, w.n, w.k, w.dtype, w.bias_layout) == (8192, 8192, 8192, W.BF16, "col")


def test_layernorm_operands():
    o = W.layernorm_operands(40, 96, W.BF16, seed=2, residual_std=0.5)
    x = W.bits_to_f32(o.x, W.BF16)
    assert o.x.shape == (40, 96) and o.gamma.shape == (96,) and o.beta.shape == (96,) and o.residual.shape == (40, 96)
    assert abs(float(x.mean()) - 0.5) < 0.1 and 0.8 < float(x.std()) < 1.2
    g = W.bits_to_f32(o.gamma, W.BF16)
    assert abs(float(g.mean()) - 1.0) < 0.05
    assert set(W.LAYERNORM_WORKLOADS) == {"layernorm_bf16_4096x1024", "layernorm_bf16_65536x16384"}
