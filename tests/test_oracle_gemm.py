"""Pins for the oracle's FP8 contraction and scale epilogue (CPU only).

  * the hand-worked example in tests/golden/ptpc_worked_example.txt;
  * exact rational brute force (Python Fractions, values decoded by PyTorch)
    on small non-square shapes -- a transposed operand or a dropped term fails;
  * the double sum equals the int64 sum of the integer units exactly, also at
    the longest K (28672) with the largest codes;
  * fused == two-step: scaling after the sum equals dequantizing first
    (vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm", §The
    challenge: two-step vs fused and §The solution: fusion).
"""
from fractions import Fraction

import numpy as np
import torch

import workloads
from conftest import read_golden


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


def test_worked_example_end_to_end(orc):
    g = read_golden("ptpc_worked_example.txt")
    x = workloads.f32_to_bf16_bits(np.array([[float(v) for v in r] for r in g["x"]], np.float32))
    w = workloads.f32_to_bf16_bits(np.array([[float(v) for v in r] for r in g["w"]], np.float32))
    r = orc.ptpc_linear(x, w)
    assert np.array_equal(r["acc"], np.array([[float(v) for v in row] for row in g["acc"]]))
    assert np.array_equal(r["ref"], np.array([[float(v) for v in row] for row in g["ref"]]))
    want = np.array([[int(v, 16) for v in row] for row in g["out_bf16"]], np.uint16)
    assert np.array_equal(r["out_bf16"], want)


def test_brute_force_fractions(orc):
    rng = np.random.default_rng(0)
    T, Ci, Co = 3, 40, 5
    qx = finite_codes(rng, (T, Ci))
    qw = finite_codes(rng, (Ci, Co))
    acc = orc.gemm_exact(qx, qw)
    dxv, dwv = torch_decode(qx), torch_decode(qw)
    for t in range(T):
        for o in range(Co):
            s = sum(Fraction(float(dxv[t, k])) * Fraction(float(dwv[k, o])) for k in range(Ci))
            assert Fraction(float(acc[t, o])) == s


def test_double_equals_int64(orc):
    rng = np.random.default_rng(1)
    qx = finite_codes(rng, (17, 1000))
    qw = finite_codes(rng, (1000, 23))
    a = orc.gemm_exact(qx, qw)
    b = orc.gemm_exact_i64(qx, qw)
    assert np.array_equal(a, b.astype(np.float64) * 2.0 ** -18)


def test_long_k_extremes_exact(orc):
    K = 28672
    qx = np.full((2, K), 0x7E, np.uint8)           # +448
    qx[1, ::2] = 0xFE                              # alternate -448
    qw = np.full((K, 3), 0x7E, np.uint8)
    qw[:, 1] = 0x01                                # 2^-9
    qw[::3, 2] = 0x81                              # -2^-9 every third row
    a = orc.gemm_exact(qx, qw)
    b = orc.gemm_exact_i64(qx, qw)
    assert a[0, 0] == K * 448.0 * 448.0
    assert a[1, 0] == 0.0
    assert a[0, 1] == K * 448.0 * 2.0 ** -9
    assert np.array_equal(a, b.astype(np.float64) * 2.0 ** -18)


def test_sampled_equals_full(orc):
    rng = np.random.default_rng(2)
    qx = finite_codes(rng, (30, 200))
    qw = finite_codes(rng, (200, 50))
    full = orc.gemm_exact(qx, qw)
    rows = rng.integers(0, 30, 100)
    cols = rng.integers(0, 50, 100)
    assert np.array_equal(orc.gemm_exact_sampled(qx, qw, rows, cols), full[rows, cols])


def test_fused_equals_two_step(orc):
    _, x, w = workloads.make("tiny")
    qx, dx = orc.quant_act(x)
    qw, dw = orc.quant_weight(w)
    two_step = orc.apply_scales(orc.gemm_exact(qx, qw), dx, dw)
    fused = orc.gemm_dequant_first(qx, dx, qw, dw)
    scale = np.abs(two_step).max()
    assert np.max(np.abs(fused - two_step)) <= 1e-12 * scale


def test_constant_scales_are_per_tensor(orc):
    """With one scale for all rows and one for all columns the output is the
    per-tensor FP8 product: acc times a single scalar."""
    rng = np.random.default_rng(3)
    v = np.clip(rng.standard_normal((12, 64)).astype(np.float32), -3.9, 3.9)
    v[:, 0] = 4.0
    u = np.clip(rng.standard_normal((64, 9)).astype(np.float32) * 0.02, -0.079, 0.079)
    u[5, :] = -0.08
    x = workloads.f32_to_bf16_bits(v)
    w = workloads.f32_to_bf16_bits(u)
    r = orc.ptpc_linear(x, w)
    qxt, sx = orc.quant_tensor(x)
    qwt, sw = orc.quant_tensor(w)
    assert np.array_equal(r["qx"], qxt) and np.array_equal(r["qw"], qwt)
    per_tensor = orc.gemm_exact(qxt, qwt) * float(sx) * float(sw)
    assert np.array_equal(r["ref"], per_tensor)


def test_per_token_per_channel_beats_per_tensor_on_outliers(orc):
    """The method's claim in miniature: with outliers in a few fixed channels
    and token magnitudes spread over three decades, per-token + per-channel
    scales keep every token's output accurate, while one scale per tensor
    pushes the quiet tokens into E4M3's subnormal range.  Measured as the
    worst per-token relative error against the exact bf16 product."""
    _, x, w = workloads.make("tiny")
    xf = workloads.bf16_bits_to_f32(x)
    xf[::3] *= np.float32(1.0 / 4096)                # quiet tokens next to loud ones
    x = workloads.f32_to_bf16_bits(xf)
    xd = workloads.bf16_bits_to_f32(x).astype(np.float64)
    wd = workloads.bf16_bits_to_f32(w).astype(np.float64)
    exact = xd @ wd
    r = orc.ptpc_linear(x, w)
    qxt, sx = orc.quant_tensor(x)
    qwt, sw = orc.quant_tensor(w)
    per_tensor = orc.gemm_exact(qxt, qwt) * float(sx) * float(sw)

    def worst_row(y):
        return float(np.max(np.linalg.norm(y - exact, axis=1) / np.linalg.norm(exact, axis=1)))

    e_ptpc, e_tensor = worst_row(r["ref"]), worst_row(per_tensor)
    assert e_ptpc < 0.1 and e_tensor > 4 * e_ptpc, (e_ptpc, e_tensor)


def test_scales_full_and_sampled_against_exact_rationals(orc):
    """The scale step ([PTPC] §Understanding the figure: Delta_X is T x 1,
    one per token row; Delta_W is 1 x Co, one per output column) on a
    non-square shape with distinct scales everywhere: every reference value,
    whole-matrix and sampled, is within double rounding of the exact rational
    acc * Delta_X[t] * Delta_W[o] computed here from PyTorch-decoded codes.
    A swapped row / column index or a scale taken from the wrong side fails."""
    rng = np.random.default_rng(5)
    T, Ci, Co = 9, 24, 5
    qx = finite_codes(rng, (T, Ci))
    qw = finite_codes(rng, (Ci, Co))
    dx = (rng.uniform(0.5, 1.0, T) * 2.0 ** rng.integers(-20, 20, T)).astype(np.float32)
    dw = (rng.uniform(0.5, 1.0, Co) * 2.0 ** rng.integers(-20, 20, Co)).astype(np.float32)
    xv, wv = torch_decode(qx), torch_decode(qw)
    exact = [[sum(Fraction(float(xv[t, k])) * Fraction(float(wv[k, o])) for k in range(Ci))
              * Fraction(float(dx[t])) * Fraction(float(dw[o])) for o in range(Co)]
             for t in range(T)]

    def close(got, want):
        return abs(Fraction(float(got)) - want) <= Fraction(2) ** -51 * abs(want)

    full = orc.apply_scales(orc.gemm_exact(qx, qw), dx, dw)
    assert full.shape == (T, Co)
    assert all(close(full[t, o], exact[t][o]) for t in range(T) for o in range(Co))
    rows = np.concatenate([np.arange(T), rng.integers(0, T, 40)])
    cols = np.concatenate([np.arange(T) % Co, rng.integers(0, Co, 40)])
    acc = orc.gemm_exact_sampled(qx, qw, rows, cols)
    ref = orc.apply_scales_sampled(acc, rows, cols, dx, dw)
    assert all(close(ref[i], exact[rows[i]][cols[i]]) for i in range(rows.size))
