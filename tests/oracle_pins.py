"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with brute force, a closed form, an invariant, a hand-derived
golden value or an independent library routine.  ``test_oracle_pins.py`` runs
them against the oracle; ``test_oracle_mutants.py`` plants mistakes in the
oracle and checks that some pin catches each one.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from egm_workloads import (BF16, E4M3, E5M2, F16, f32_to_fp8_bits, fp8_integer_operands, fp8_operands,
                           gemm_operands, integer_operands)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _frac_of_bits(bits, dtype, o):
    # exact rational value of each 16-bit pattern, taken from float.as_integer_ratio
    return [[Fraction(*float(v).as_integer_ratio()) for v in row] for row in o.widen(bits, dtype)]


def _brute(a, b, bias, layout, r, epilog):
    """Exact rational GEMM + epilogue by three nested loops (no GELU)."""
    m, k = len(a), len(a[0]) if a and a[0] else 0
    n = len(b[0]) if b else (len(r[0]) if r else 0)
    y, z = [], []
    for i in range(m):
        yr, zr = [], []
        for j in range(n):
            s = Fraction(0)
            for t in range(k):
                s += a[i][t] * b[t][j]
            if epilog != "DEFAULT":
                s += bias[i] if layout == "row" else bias[j]
            zr.append(s)
            if epilog in ("RELU_BIAS", "RELU_AUX_BIAS"):
                yr.append(s if s > 0 else Fraction(0))
            elif epilog == "BIAS_RESIDUAL":
                yr.append(s + r[i][j])
            else:
                yr.append(s)
        y.append(yr)
        z.append(zr)
    return y, z


# ---------------------------------------------------------------------------
def pin_brute_force_fraction(o):
    """Exact rational brute force on tiny shapes, every epilog but GELU."""
    shapes = [(1, 8, 1), (2, 8, 3), (3, 16, 5), (5, 8, 8), (8, 24, 17), (17, 8, 2)]
    for s, (m, n, k) in enumerate(shapes):
        for dtype in (F16, BF16):
            for layout in ("row", "col"):
                ops = gemm_operands(m, n, k, dtype, seed=100 + s, a_std=1.3, b_std=0.7,
                                    bias_layout=layout, bias_std=0.5, residual_std=0.9)
                a = _frac_of_bits(ops.a, dtype, o)
                b = _frac_of_bits(ops.b, dtype, o)
                bias = _frac_of_bits(ops.bias[None, :], dtype, o)[0]
                r = _frac_of_bits(ops.residual, dtype, o)
                for ep in ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL"):
                    y, z, mask = o.reference(ops.a, ops.b, dtype, ep, ops.bias, layout,
                                             ops.residual if ep == "BIAS_RESIDUAL" else None)
                    ye, ze = _brute(a, b, bias, layout, r, ep)
                    for i in range(m):
                        for j in range(n):
                            ex = float(ye[i][j])
                            assert abs(y[i, j] - ex) <= 1e-12 * (1.0 + abs(ex)), (ep, dtype, layout, i, j)
                    if ep == "RELU_AUX_BIAS":
                        for i in range(m):
                            for j in range(n):
                                bit = (int(mask[i, j // 8]) >> (j % 8)) & 1
                                assert bit == (1 if ze[i][j] > 0 else 0), (i, j)


def pin_integer_exact(o):
    """Small-integer operands: P equals the int64 matmul exactly."""
    for dtype in (F16, BF16):
        for (m, n, k) in [(33, 40, 64), (7, 8, 1), (64, 64, 16)]:
            ops = integer_operands(m, n, k, dtype, seed=7, bias_layout="col")
            ai = o.widen(ops.a, dtype).astype(np.int64)
            bi = o.widen(ops.b, dtype).astype(np.int64)
            y, _, _ = o.reference(ops.a, ops.b, dtype, "DEFAULT")
            assert np.array_equal(y, (ai @ bi).astype(np.float64))
            bb = o.widen(ops.bias, dtype).astype(np.int64)
            y, _, _ = o.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, "col")
            assert np.array_equal(y, (ai @ bi + bb[None, :]).astype(np.float64))


def pin_identity_a(o):
    """A = I (m = k): D = B + bias."""
    for dtype in (F16, BF16):
        n, k = 24, 16
        eye = o.round_to_bits(np.eye(k), dtype)
        ops = gemm_operands(k, n, k, dtype, seed=3, bias_layout="row")
        y, _, _ = o.reference(eye, ops.b, dtype, "BIAS", ops.bias, "row")
        expect = o.widen(ops.b, dtype) + o.widen(ops.bias, dtype)[:, None]
        assert np.array_equal(y, expect)
        y, _, _ = o.reference(eye, ops.b, dtype, "DEFAULT")
        assert np.array_equal(y, o.widen(ops.b, dtype))


def pin_zero_b_gives_bias(o):
    """B = 0: Z is the bias broadcast (row: constant along a row; col: along a column)."""
    for dtype in (F16, BF16):
        m, n, k = 9, 16, 8
        ops = gemm_operands(m, n, k, dtype, seed=4, bias_layout="row", residual_std=1.0)
        zb = np.zeros((k, n), np.uint16)
        bias = o.widen(ops.bias, dtype)
        y, _, _ = o.reference(ops.a, zb, dtype, "BIAS", ops.bias, "row")
        assert np.array_equal(y, np.repeat(bias[:, None], n, axis=1))
        colb = gemm_operands(m, n, k, dtype, seed=5, bias_layout="col").bias
        y, _, _ = o.reference(ops.a, zb, dtype, "BIAS", colb, "col")
        assert np.array_equal(y, np.repeat(o.widen(colb, dtype)[None, :], m, axis=0))
        y, _, _ = o.reference(ops.a, zb, dtype, "BIAS_RESIDUAL", ops.bias, "row", ops.residual)
        assert np.array_equal(y, bias[:, None] + o.widen(ops.residual, dtype))


def pin_zero_bias_is_default(o):
    for dtype in (F16, BF16):
        ops = gemm_operands(12, 16, 40, dtype, seed=6, bias_layout="col")
        zero = np.zeros(16, np.uint16)
        y0, _, _ = o.reference(ops.a, ops.b, dtype, "DEFAULT")
        y1, _, _ = o.reference(ops.a, ops.b, dtype, "BIAS", zero, "col")
        assert np.array_equal(y0, y1)
        assert np.allclose(y0, o.widen(ops.a, dtype) @ o.widen(ops.b, dtype), rtol=0, atol=1e-12)


def pin_transpose_duality(o):
    """epi(A.B + b_row) == epi(B^T.A^T + b_col)^T ties the row and column layouts."""
    for dtype in (F16, BF16):
        m, n, k = 16, 24, 32
        ops = gemm_operands(m, n, k, dtype, seed=8, bias_layout="row")
        for ep in ("BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS"):
            y1, z1, _ = o.reference(ops.a, ops.b, dtype, ep, ops.bias, "row")
            y2, z2, _ = o.reference(np.ascontiguousarray(ops.b.T), np.ascontiguousarray(ops.a.T),
                                    dtype, ep, ops.bias, "col")
            assert np.allclose(y1, y2.T, rtol=0, atol=1e-12), ep
            assert np.allclose(z1, z2.T, rtol=0, atol=1e-12), ep


def pin_relu_invariants(o):
    for dtype in (F16, BF16):
        ops = gemm_operands(40, 48, 64, dtype, seed=9, a_std=1.0, bias_layout="col")
        for ep in ("RELU_BIAS", "RELU_AUX_BIAS"):
            y, z, _ = o.reference(ops.a, ops.b, dtype, ep, ops.bias, "col")
            assert (y >= 0).all()
            assert (y[z < 0] == 0).all()
            assert np.array_equal(y[z > 0], z[z > 0])
            assert (z < 0).any() and (z > 0).any()


def pin_mask_golden_bit_order(o):
    """Z[i,j] = j - i through the real path: A[i] = (1, i), B = [[j...], [-1...]]."""
    golden = {}
    with open(os.path.join(GOLDEN, "relu_mask_j_minus_i.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                i, b0, b1 = line.split()
                golden[int(i)] = (int(b0, 16), int(b1, 16))
    m, n = 16, 16
    for dtype in (F16, BF16):
        a = o.round_to_bits(np.stack([np.ones(m), np.arange(m)], axis=1), dtype)
        b = o.round_to_bits(np.stack([np.arange(n), -np.ones(n)], axis=0), dtype)
        zero = np.zeros(n, np.uint16)
        _, z, mask = o.reference(a, b, dtype, "RELU_AUX_BIAS", zero, "col")
        assert np.array_equal(z, np.arange(n)[None, :] - np.arange(m)[:, None])
        assert mask.shape == (m, n // 8) and mask.dtype == np.uint8
        for i, (b0, b1) in golden.items():
            assert (int(mask[i, 0]), int(mask[i, 1])) == (b0, b1), i


def pin_mask_popcount(o):
    for dtype in (F16, BF16):
        ops = gemm_operands(32, 64, 48, dtype, seed=10, bias_layout="row")
        y, z, mask = o.reference(ops.a, ops.b, dtype, "RELU_AUX_BIAS", ops.bias, "row")
        pop = int(np.unpackbits(mask).sum())
        assert pop == int((y > 0).sum()) == int((z > 0).sum())
        # each row's bits, read LSB-first one byte at a time, are the row's predicate
        for i in range(0, 32, 7):
            bits = [(int(mask[i, j >> 3]) >> (j & 7)) & 1 for j in range(64)]
            assert bits == [int(v > 0) for v in z[i]]


def pin_gelu_library(o):
    """tanh-form GELU against torch's own (CPU, float64) and closed forms."""
    import torch
    x = np.concatenate([np.linspace(-12, 12, 4001), [-40.0, -1e-8, 0.0, 1e-8, 40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x.copy()), approximate="tanh").numpy()
    got = o.gelu_tanh(x)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-15)
    assert o.gelu_tanh(np.array([0.0]))[0] == 0.0
    # odd part: gelu(z) - gelu(-z) = z  (since tanh is odd)
    z = np.linspace(-6, 6, 1001)
    assert np.allclose(o.gelu_tanh(z) - o.gelu_tanh(-z), z, rtol=0, atol=1e-13)
    # asymptotes
    assert abs(o.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(o.gelu_tanh(np.array([-30.0]))[0]) < 1e-12
    # the epilog applies it to Z = P + bias
    ops = gemm_operands(8, 16, 16, BF16, seed=11, bias_layout="col")
    y, z, _ = o.reference(ops.a, ops.b, BF16, "GELU_BIAS", ops.bias, "col")
    assert np.allclose(y, torch.nn.functional.gelu(torch.from_numpy(z.copy()), approximate="tanh").numpy(),
                       rtol=1e-14, atol=1e-15)


def pin_gelu_math_tanh(o):
    """Elementwise against math.tanh (the C library) on exact Z from brute force."""
    ops = gemm_operands(3, 8, 5, F16, seed=12, a_std=2.0, b_std=1.0, bias_layout="row")
    a = _frac_of_bits(ops.a, F16, o)
    b = _frac_of_bits(ops.b, F16, o)
    bias = _frac_of_bits(ops.bias[None, :], F16, o)[0]
    _, ze = _brute(a, b, bias, "row", None, "BIAS")
    y, _, _ = o.reference(ops.a, ops.b, F16, "GELU_BIAS", ops.bias, "row")
    c = math.sqrt(2.0 / math.pi)
    for i in range(3):
        for j in range(8):
            zz = float(ze[i][j])
            ex = 0.5 * zz * (1.0 + math.tanh(c * (zz + 0.044715 * zz ** 3)))
            assert abs(y[i, j] - ex) <= 1e-13 * (1 + abs(ex))


def pin_residual(o):
    for dtype in (F16, BF16):
        ops = gemm_operands(16, 32, 24, dtype, seed=13, bias_layout="col", residual_std=1.0)
        zero_r = np.zeros_like(ops.residual)
        y0, _, _ = o.reference(ops.a, ops.b, dtype, "BIAS", ops.bias, "col")
        y1, _, _ = o.reference(ops.a, ops.b, dtype, "BIAS_RESIDUAL", ops.bias, "col", zero_r)
        assert np.array_equal(y0, y1)
        y2, _, _ = o.reference(ops.a, ops.b, dtype, "BIAS_RESIDUAL", ops.bias, "col", ops.residual)
        assert np.allclose(y2 - y0, o.widen(ops.residual, dtype), rtol=0, atol=1e-12)


def pin_row_subset(o):
    ops = gemm_operands(64, 32, 48, F16, seed=14, bias_layout="row", residual_std=1.0)
    rows = np.array([0, 5, 17, 63])
    for ep in ("BIAS", "BIAS_RESIDUAL", "RELU_AUX_BIAS"):
        r = ops.residual if ep == "BIAS_RESIDUAL" else None
        yf, zf, mf = o.reference(ops.a, ops.b, F16, ep, ops.bias, "row", r)
        ys, zs, ms = o.reference(ops.a, ops.b, F16, ep, ops.bias, "row", r, rows=rows)
        assert np.array_equal(ys, yf[rows]) and np.array_equal(zs, zf[rows])
        if mf is not None:
            assert np.array_equal(ms, mf[rows])


def pin_rounding_golden(o):
    with open(os.path.join(GOLDEN, "rounding_cases.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            dtype, val, bits = line.split()[:3]
            got = int(o.round_to_bits(np.array([float.fromhex(val)]), dtype)[0])
            assert got == int(bits, 16), (dtype, val, hex(got), bits)


def pin_rounding_library(o):
    """fp16: numpy's double->half cast; bf16: torch's float->bfloat16 cast on
    values exact in fp32 (so torch's single rounding is the same rounding)."""
    import torch
    g = np.random.default_rng(15)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-6, 1e-3, 1, 30, 3e4)])
    # exact fp16 midpoints and their neighbours
    h = g.standard_normal(5000).astype(np.float16).astype(np.float64)
    hn = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mid = (h + hn) / 2
    x = np.concatenate([x, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])
    assert np.array_equal(o.round_to_bits(x, F16), x.astype(np.float16).view(np.uint16))
    xf = np.concatenate([g.standard_normal(20000).astype(np.float32),
                         (g.standard_normal(20000) * 1e-30).astype(np.float32)])
    # exact bf16 midpoints (representable in fp32)
    bb = torch.from_numpy(xf.copy()).to(torch.bfloat16)
    up = torch.nextafter(bb, torch.tensor(float("inf"), dtype=torch.bfloat16))
    mids = ((bb.float() + up.float()) / 2).numpy()
    xf = np.concatenate([xf, mids])
    want = torch.from_numpy(xf.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.round_to_bits(xf.astype(np.float64), BF16), want)


def pin_widen_exhaustive(o):
    """Every fp16 / bf16 pattern widens to the value numpy / torch give it."""
    import torch
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = o.widen(allb, F16)
    ref = allb.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin], ref[fin])
    w = o.widen(allb, BF16)
    ref = torch.from_numpy(allb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin], ref[fin])


def pin_empty_k(o):
    """K = 0: the product is zero, D = epilogue(bias)."""
    a = np.zeros((4, 0), np.uint16)
    b = np.zeros((0, 8), np.uint16)
    bias = o.round_to_bits(np.array([-1.0, 0.0, 2.0, 3.5]), F16)
    y, z, mask = o.reference(a, b, F16, "RELU_AUX_BIAS", bias, "row")
    assert np.array_equal(y, np.repeat(np.array([[0.0], [0.0], [2.0], [3.5]]), 8, axis=1))
    assert list(mask[:, 0]) == [0, 0, 255, 255]


# ---------------------------------------------------------------------------
# backward: DRELU / DRELU_BGRAD
# ---------------------------------------------------------------------------
def _golden_backward():
    rows = {}
    with open(os.path.join(GOLDEN, "drelu_bgrad_small.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                rows.setdefault(key, []).append([float(v) for v in vals])
    return rows


def pin_backward_golden(o):
    """The hand-derived example in tests/golden/drelu_bgrad_small.txt, through
    the whole backward path (A = dY, B = I)."""
    g = _golden_backward()
    a = o.round_to_bits(np.array(g["A"]), F16)
    b = o.round_to_bits(np.eye(8), F16)
    mask = np.array(g["MASK"], dtype=np.uint8).reshape(2, 1)
    dz, dcol, _ = o.backward_reference(a, b, F16, "DRELU_BGRAD", mask, "col")
    assert np.array_equal(dz, np.array(g["DZ"]))
    assert np.array_equal(dcol, np.array(g["DBIAS_COL"][0]))
    _, drow, _ = o.backward_reference(a, b, F16, "DRELU_BGRAD", mask, "row")
    assert np.array_equal(drow, np.array(g["DBIAS_ROW"][0]))
    dz2, none, _ = o.backward_reference(a, b, F16, "DRELU", mask)
    assert none is None and np.array_equal(dz2, dz)


def pin_backward_brute_force(o):
    """Exact rational brute force: dZ[i][j] = (sum_t a b) if bit j of row i, and
    the bias gradients as plain loops over Fractions."""
    rng = np.random.default_rng(7)
    for s, (m, n, k) in enumerate([(1, 8, 3), (3, 16, 5), (5, 24, 9), (9, 8, 2)]):
        for dtype in (F16, BF16):
            ops = gemm_operands(m, n, k, dtype, seed=300 + s, a_std=1.1, b_std=0.8, bias_layout="col")
            mask = rng.integers(0, 256, size=(m, n // 8), dtype=np.uint8)
            fa, fb = _frac_of_bits(ops.a, dtype, o), _frac_of_bits(ops.b, dtype, o)
            dz_ex = [[Fraction(0)] * n for _ in range(m)]
            for i in range(m):
                for j in range(n):
                    if (int(mask[i, j // 8]) >> (j % 8)) & 1:
                        dz_ex[i][j] = sum((fa[i][t] * fb[t][j] for t in range(k)), Fraction(0))
            dz, dcol, _ = o.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, "col")
            _, drow, _ = o.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, "row")
            for i in range(m):
                for j in range(n):
                    assert abs(dz[i, j] - float(dz_ex[i][j])) <= 1e-12
            for j in range(n):
                assert abs(dcol[j] - float(sum((dz_ex[i][j] for i in range(m)), Fraction(0)))) <= 1e-11
            for i in range(m):
                assert abs(drow[i] - float(sum(dz_ex[i], Fraction(0)))) <= 1e-11


def pin_drelu_is_relu_derivative(o):
    """With the mask the forward pass packed from Z, DRELU(dY) equals the
    directional derivative of ReLU at Z along dY: (relu(Z + h dY) - relu(Z)) / h
    for a step h too small to flip any sign (|Z| >= 1/8, |h dY| < 1/64)."""
    rng = np.random.default_rng(11)
    m, n = 6, 24
    # dyadic values, so z + h dy and the difference quotient are exact in fp64
    z = rng.choice([-1.0, 1.0], size=(m, n)) * rng.integers(1, 17, size=(m, n)) / 8.0
    dy = rng.integers(-3, 4, size=(m, n)).astype(np.float64)
    h = 2.0 ** -8
    fd = (o.relu(z + h * dy) - o.relu(z)) / h
    assert np.array_equal(o.drelu(dy, o.relu_mask(z)), fd)


def pin_drelu_all_or_nothing(o):
    """A full mask keeps the product (DRELU = DEFAULT); an empty one gives 0."""
    ops = gemm_operands(40, 32, 24, BF16, seed=21, bias_layout="col")
    p = o.product(o.widen(ops.a, BF16), o.widen(ops.b, BF16))
    full = np.full((40, 4), 255, dtype=np.uint8)
    dz, _, _ = o.backward_reference(ops.a, ops.b, BF16, "DRELU", full)
    assert np.array_equal(dz, p)
    dz0, dcol, _ = o.backward_reference(ops.a, ops.b, BF16, "DRELU_BGRAD", np.zeros_like(full), "col")
    assert not dz0.any() and not dcol.any()


def pin_bias_grad_invariants(o):
    """Both gradients sum to the sum of dZ; the row and column gradients are
    each other's transpose; integer inputs give integer sums exactly."""
    ops = integer_operands(33, 40, 16, F16, seed=5)
    rng = np.random.default_rng(3)
    mask = rng.integers(0, 256, size=(33, 5), dtype=np.uint8)
    dz, dcol, _ = o.backward_reference(ops.a, ops.b, F16, "DRELU_BGRAD", mask, "col")
    _, drow, _ = o.backward_reference(ops.a, ops.b, F16, "DRELU_BGRAD", mask, "row")
    assert dcol.sum() == drow.sum() == dz.sum()
    assert np.array_equal(o.bias_grad(dz.T, "row"), dcol)
    ai = o.widen(ops.a, F16).astype(np.int64)
    bi = o.widen(ops.b, F16).astype(np.int64)
    keep = np.unpackbits(mask, axis=1, bitorder="little").astype(bool)
    want = np.where(keep, ai @ bi, 0)
    assert np.array_equal(dz, want) and np.array_equal(dcol, want.sum(axis=0)) and np.array_equal(drow, want.sum(axis=1))


def pin_bias_grad_error_bound(o):
    """The bound covers an actual fp32 computation (fp32 dot products, then an
    fp32 running sum) and is not vacuous (a small multiple of the error)."""
    for dtype in (F16, BF16):
        ops = gemm_operands(300, 64, 512, dtype, seed=9, a_std=1.0, b_std=1.0 / math.sqrt(512), bias_layout="col")
        rng = np.random.default_rng(4)
        mask = rng.integers(0, 256, size=(300, 8), dtype=np.uint8)
        dz, dcol, bound = o.backward_reference(ops.a, ops.b, dtype, "DRELU_BGRAD", mask, "col")
        p32 = np.zeros((300, 64), dtype=np.float32)
        a32, b32 = o.widen(ops.a, dtype).astype(np.float32), o.widen(ops.b, dtype).astype(np.float32)
        for t in range(512):  # one rounding per step, as a sequential fp32 dot product
            p32 = (p32 + a32[:, t:t + 1] * b32[t:t + 1, :]).astype(np.float32)
        keep = np.unpackbits(mask, axis=1, bitorder="little").astype(bool)
        dz32 = np.where(keep, p32, np.float32(0))
        s32 = np.zeros(64, dtype=np.float32)
        for i in range(300):
            s32 = (s32 + dz32[i]).astype(np.float32)
        err = np.abs(s32.astype(np.float64) - dcol)
        assert (err <= bound).all() and (bound > 0).all()
    # closed form: A and B all ones, full mask: |A|.|B| = K everywhere, so the
    # (1,n) gradient's bound is (K + M) u M K and the (m,1) one's (K + N) u N K
    m, n, k = 24, 16, 40
    ones_a = o.round_to_bits(np.ones((m, k)), F16)
    ones_b = o.round_to_bits(np.ones((k, n)), F16)
    full = np.full((m, n // 8), 255, dtype=np.uint8)
    _, _, bcol = o.backward_reference(ones_a, ones_b, F16, "DRELU_BGRAD", full, "col")
    _, _, brow = o.backward_reference(ones_a, ones_b, F16, "DRELU_BGRAD", full, "row")
    assert np.allclose(bcol, (k + m) * 2.0 ** -24 * m * k, rtol=1e-15, atol=0)
    assert np.allclose(brow, (k + n) * 2.0 ** -24 * n * k, rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# fp8 operands
# ---------------------------------------------------------------------------
def _parse_hexfloat(t):
    if t in ("inf", "-inf", "nan"):
        return float(t)
    return float.fromhex(t)


def pin_fp8_decode_golden(o):
    """Hand-derived values of selected patterns (tests/golden/fp8_values.txt)."""
    n = 0
    with open(os.path.join(GOLDEN, "fp8_values.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            fmt, bits, val = line.split()[:3]
            got = float(o.decode_fp8(np.array([int(bits, 16)], dtype=np.uint8), fmt)[0])
            want = _parse_hexfloat(val)
            if math.isnan(want):
                assert math.isnan(got), (fmt, bits, got)
            else:
                assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (fmt, bits, got, want)
            n += 1
    assert n >= 20


def pin_fp8_decode_library(o):
    """All 256 patterns of both formats against torch's fp8 -> fp32 conversion."""
    import torch
    bits = np.arange(256, dtype=np.uint8)
    for fmt, tdt in ((E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)):
        mine = o.decode_fp8(bits, fmt)
        ref = torch.from_numpy(bits).view(tdt).float().double().numpy()
        assert np.array_equal(np.isnan(mine), np.isnan(ref)), fmt
        ok = ~np.isnan(ref)
        assert np.array_equal(mine[ok], ref[ok]), fmt
        assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok])), fmt


def pin_fp8_e5m2_is_fp16_high_byte(o):
    """E5M2 has fp16's sign and exponent fields and its two top mantissa bits,
    so a pattern followed by a zero byte is the same number in fp16."""
    bits = np.arange(256, dtype=np.uint8)
    as_f16 = (bits.astype(np.uint16) << np.uint16(8)).view(np.float16).astype(np.float64)
    mine = o.decode_fp8(bits, E5M2)
    ok = ~np.isnan(as_f16)
    assert np.array_equal(np.isnan(mine), ~ok) and np.array_equal(mine[ok], as_f16[ok])


def pin_fp8_brute_force(o):
    """Exact rational brute force, every format pair and epilog but GELU, with
    non-trivial fp32 scales: Z = sa sb sum(a b) + bias."""
    shapes = [(1, 8, 1), (3, 16, 5), (5, 8, 9), (9, 24, 4)]
    pairs = [(E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]
    for s, (m, n, k) in enumerate(shapes):
        for pi, (fa, fb) in enumerate(pairs):
            out = BF16 if (s + pi) % 2 else F16
            layout = "row" if pi % 2 else "col"
            ops = fp8_operands(m, n, k, fa, fb, out, seed=500 + 4 * s + pi, a_std=1.2, b_std=0.9,
                               bias_layout=layout, bias_std=0.5, residual_std=0.7)
            scale = Fraction(*float(ops.scale_a).as_integer_ratio()) * Fraction(*float(ops.scale_b).as_integer_ratio())
            fa_ = [[Fraction(*float(v).as_integer_ratio()) * scale for v in row] for row in o.decode_fp8(ops.a, fa)]
            fb_ = [[Fraction(*float(v).as_integer_ratio()) for v in row] for row in o.decode_fp8(ops.b, fb)]
            bias = [Fraction(*float(v).as_integer_ratio()) for v in o.widen(ops.bias, out)]
            r = _frac_of_bits(ops.residual, out, o)
            for epilog in ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "BIAS_RESIDUAL"):
                y_ex, z_ex = _brute(fa_, fb_, bias, layout, r, epilog)
                y, z, mask = o.reference_fp8(ops.a, ops.b, fa, fb, ops.scale_a, ops.scale_b, out, epilog,
                                             ops.bias, layout, ops.residual)
                for i in range(m):
                    for j in range(n):
                        assert abs(y[i, j] - float(y_ex[i][j])) <= 1e-12 * (1 + abs(float(y_ex[i][j]))), (epilog, i, j)
                if epilog == "RELU_AUX_BIAS":
                    want = np.packbits(np.array([[zz > 0 for zz in row] for row in z_ex]), axis=1, bitorder="little")
                    assert np.array_equal(mask, want)


def pin_fp8_matches_16bit_path(o):
    """With unit scales, fp8 operands give the 16-bit path's result on the
    same values: every E4M3 / E5M2 value is exact in fp16 and bf16 (the 16-bit
    patterns come from torch's conversion, or from the E5M2 byte shifted into
    fp16's high byte)."""
    import torch
    for fmt in (E4M3, E5M2):
        for out in (F16, BF16):
            ops = fp8_operands(12, 24, 40, fmt, fmt, out, seed=77, a_std=1.0, b_std=0.3, bias_layout="col")
            one = np.float32(1.0)
            tdt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
            to16 = torch.float16 if out == F16 else torch.bfloat16
            if fmt == E5M2 and out == F16:
                a16 = ops.a.astype(np.uint16) << np.uint16(8)
                b16 = ops.b.astype(np.uint16) << np.uint16(8)
            else:
                a16 = torch.from_numpy(ops.a).view(tdt).to(to16).view(torch.int16).numpy().view(np.uint16)
                b16 = torch.from_numpy(ops.b).view(tdt).to(to16).view(torch.int16).numpy().view(np.uint16)
            for epilog in ("DEFAULT", "BIAS", "GELU_BIAS", "RELU_AUX_BIAS"):
                y8, z8, m8 = o.reference_fp8(ops.a, ops.b, fmt, fmt, one, one, out, epilog, ops.bias, "col")
                y16, z16, m16 = o.reference(a16, b16, out, epilog, ops.bias, "col")
                assert np.array_equal(y8, y16) and np.array_equal(z8, z16), (fmt, out, epilog)
                assert (m8 is None and m16 is None) or np.array_equal(m8, m16)


def pin_fp8_scales(o):
    """Power-of-two scales scale the product exactly and never the bias; the
    two scales enter only through their product; integer operands give exact
    integers."""
    ops = fp8_integer_operands(16, 32, 24, E4M3, E5M2, BF16, seed=3, bias_layout="row")
    one = np.float32(1.0)
    y1, _, _ = o.reference_fp8(ops.a, ops.b, E4M3, E5M2, one, one, BF16, "DEFAULT")
    ai = o.decode_fp8(ops.a, E4M3).astype(np.int64)
    bi = o.decode_fp8(ops.b, E5M2).astype(np.int64)
    assert np.array_equal(y1, ai @ bi)
    y2, _, _ = o.reference_fp8(ops.a, ops.b, E4M3, E5M2, np.float32(8.0), np.float32(0.25), BF16, "DEFAULT")
    assert np.array_equal(y2, 2.0 * y1)
    sa, sb = np.float32(0.3), np.float32(1.7)
    y3, _, _ = o.reference_fp8(ops.a, ops.b, E4M3, E5M2, sa, sb, BF16, "DEFAULT")
    y4, _, _ = o.reference_fp8(ops.a, ops.b, E4M3, E5M2, sb, sa, BF16, "DEFAULT")
    assert np.array_equal(y3, y4)
    assert np.allclose(y3, y1 * (float(sa) * float(sb)), rtol=1e-15, atol=0)
    # a zero B leaves the bias alone, whatever the scales
    zb = f32_to_fp8_bits(np.zeros((24, 32), dtype=np.float32), E5M2)
    y5, _, _ = o.reference_fp8(ops.a, zb, E4M3, E5M2, np.float32(3.0), np.float32(5.0), BF16, "BIAS",
                               ops.bias, "row")
    assert np.array_equal(y5, np.repeat(o.widen(ops.bias, BF16)[:, None], 32, axis=1))


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------
def _golden_layernorm():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "layernorm_small.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "CASE":
                cur = {"name": vals[0], "eps": float(vals[1])}
                cases.append(cur)
            else:
                cur[key] = np.array([float(v) for v in vals])
    return cases


def pin_layernorm_golden(o):
    cases = _golden_layernorm()
    assert len(cases) >= 6
    for c in cases:
        y, _, _ = o.layer_norm(c["X"][None, :], c["GAMMA"], c["BETA"], c["eps"],
                               c["R"][None, :] if "R" in c else None)
        assert np.array_equal(y[0], c["Y"]), (c["name"], y[0], c["Y"])


def pin_layernorm_library(o):
    """torch.nn.functional.layer_norm in fp64 (an independent implementation)."""
    import torch
    rng = np.random.default_rng(12)
    for n in (8, 100, 1024):
        x = rng.standard_normal((7, n)) * 3 + 1
        g, b = rng.standard_normal(n), rng.standard_normal(n)
        for eps in (1e-5, 0.5):
            y, mean, rstd = o.layer_norm(x, g, b, eps)
            ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (n,), torch.from_numpy(g), torch.from_numpy(b),
                                                 eps).numpy()
            assert np.allclose(y, ref, rtol=0, atol=1e-12)
            assert np.allclose(mean, x.mean(axis=1), rtol=0, atol=1e-13)
            assert np.allclose(rstd, 1 / np.sqrt(x.var(axis=1) + eps), rtol=1e-13, atol=0)


def pin_layernorm_brute_force(o):
    """Exact rational mean and variance by loops; one final square root."""
    rng = np.random.default_rng(13)
    for n in (3, 8, 17):
        x = rng.integers(-20, 21, size=(4, n)) / 8.0
        g, b = rng.integers(-8, 9, size=n) / 4.0, rng.integers(-8, 9, size=n) / 4.0
        y, mean, rstd = o.layer_norm(x, g, b, 0.0625)
        for i in range(4):
            xs = [Fraction(*float(v).as_integer_ratio()) for v in x[i]]
            mu = sum(xs, Fraction(0)) / n
            var = sum(((v - mu) ** 2 for v in xs), Fraction(0)) / n
            rs = 1.0 / math.sqrt(float(var + Fraction(1, 16)))
            assert float(mu) == mean[i] and abs(rstd[i] - rs) <= 1e-15 * rs
            for j in range(n):
                want = float(xs[j] - mu) * rs * float(g[j]) + float(b[j])
                assert abs(y[i, j] - want) <= 1e-13 * (1 + abs(want))


def pin_layernorm_invariants(o):
    """Shift invariance; scale invariance at eps = 0; the normalised row has
    mean 0 and variance var / (var + eps); gamma, beta and the residual act
    affinely."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 64))
    y0, _, _ = o.layer_norm(x, None, None, 1e-5)
    y1, _, _ = o.layer_norm(x + 7.0, None, None, 1e-5)
    assert np.allclose(y0, y1, rtol=0, atol=1e-12)
    ya, _, _ = o.layer_norm(x, None, None, 0.0)
    yb, _, _ = o.layer_norm(x * 3.5, None, None, 0.0)
    assert np.allclose(ya, yb, rtol=0, atol=1e-12)
    var = x.var(axis=1)
    assert np.allclose(y0.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose(y0.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    g, b, r = rng.standard_normal(64), rng.standard_normal(64), rng.standard_normal((5, 64))
    yg, _, _ = o.layer_norm(x, g, b, 1e-5, r)
    assert np.allclose(yg, y0 * g[None, :] + b[None, :] + r, rtol=0, atol=1e-12)


def _golden_ulps():
    rows = []
    with open(os.path.join(GOLDEN, "ulp_spacings.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                dt, v, q, *_ = line.split()
                rows.append((dt, float.fromhex(v), float.fromhex(q)))
    return rows


def pin_ulp_golden(o):
    """Hand-derived spacings of binary16 and bfloat16 (tests/golden), at either
    sign of the value."""
    rows = _golden_ulps()
    assert len(rows) >= 16 and {r[0] for r in rows} == {F16, BF16}
    for dt, v, q in rows:
        got = o.ulp(np.array([v, -v]), dt)
        assert np.array_equal(got, np.array([q, q])), (dt, v.hex(), [float(g).hex() for g in got], q.hex())


def pin_ulp_library(o):
    """Every finite value of each format, zero included, against numpy's
    spacing: np.spacing of the fp16 value itself, and for bfloat16 (the upper
    half of a binary32 whose low 16 bits are zero) the binary32 spacing times
    2^16, since both share the exponent range and bfloat16 keeps 16 fewer
    fraction bits.  Zero has the subnormal spacing."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    # numpy steps past the largest finite value to infinity; the golden file
    # holds the spacing there
    fin = np.isfinite(h) & (np.abs(h) < np.float16(65504))
    want = np.abs(np.spacing(np.abs(h[fin]))).astype(np.float64)
    assert np.array_equal(o.ulp(h[fin].astype(np.float64), F16), want)
    f = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    fin = np.isfinite(f) & (np.abs(f) < np.float32(float.fromhex("0x1.fep127")))
    want = np.abs(np.spacing(np.abs(f[fin]))).astype(np.float64) * 65536.0
    assert np.array_equal(o.ulp(f[fin].astype(np.float64), BF16), want)


def _bits_of(values, dtype):
    """Exactly representable values -> 16-bit patterns, by numpy's own casts
    (a binary16 array, or the upper half of a binary32)."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == F16:
        h = v.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), v)
        return h.view(np.uint16)
    f = v.astype(np.float32)
    b = f.view(np.uint32)
    assert np.array_equal(f.astype(np.float64), v) and not np.any(b & np.uint32(0xFFFF))
    return (b >> np.uint32(16)).astype(np.uint16)


def pin_layernorm_reference_golden(o):
    """The 16-bit entry point of the LayerNorm oracle on the hand-worked rows,
    passed as bit patterns in both formats: x, gamma, beta and the residual must
    each land in its own place."""
    cases = _golden_layernorm()
    for dtype in (F16, BF16):
        for c in cases:
            rb = _bits_of(c["R"], dtype)[None, :] if "R" in c else None
            y, mean, rstd = o.layer_norm_reference(_bits_of(c["X"], dtype)[None, :], dtype,
                                                   _bits_of(c["GAMMA"], dtype), _bits_of(c["BETA"], dtype),
                                                   c["eps"], rb)
            assert np.array_equal(y[0], c["Y"]), (dtype, c["name"], y[0], c["Y"])
            assert mean[0] == c["X"].mean()
        # gamma and beta omitted mean 1 and 0
        c = cases[0]
        y, _, _ = o.layer_norm_reference(_bits_of(c["X"], dtype)[None, :], dtype, None, None, c["eps"])
        assert np.array_equal(y[0], c["Y"])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
