"""Pins for the oracle's per-token / per-channel quantizers (CPU only).

What the pages fix (vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD
ROCm", §PTPC: a precision-targeted scheme and §Understanding the figure):
one scale per token (row of X, shape T x 1), one per weight column (shape
1 x Co), and per-tensor FP8 as the case of a single scalar scale.  Checked
here by properties that do not restate the oracle's formulas:
  * the amax element of every row/column encodes to +-448;
  * the scale is the fp32 value nearest to amax/448 (exact rational check);
  * power-of-two scaling and negation equivariance;
  * the E4M3 error bound;
  * rows sharing one amax reproduce per-tensor FP8, and with amax 448
    (scale 1) the codes equal PyTorch's direct float8 cast;
  * the weight quantizer is the activation quantizer on W transposed.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from conftest import read_golden

F32 = np.float32


def f32(b):
    return workloads.bf16_bits_to_f32(b)


def nearest_f32(fr: Fraction) -> np.float32:
    """fp32 value nearest to an exact rational (ties to even), brute force
    over the float32 neighbours of its float64 approximation."""
    c = np.float32(float(fr))
    cands = [np.nextafter(np.nextafter(c, F32(-np.inf)), F32(-np.inf)),
             np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf)),
             np.nextafter(np.nextafter(c, F32(np.inf)), F32(np.inf))]
    errs = [abs(Fraction(float(v)) - fr) for v in cands]
    best = min(errs)
    tied = [v for v, e in zip(cands, errs) if e == best]
    if len(tied) == 1:
        return tied[0]
    return [v for v in tied if (np.float32(v).view(np.uint32) & 1) == 0][0]


@pytest.fixture(scope="module")
def cfg2():
    return workloads.make("8b_qkv_decode")


def test_worked_example(orc):
    g = read_golden("ptpc_worked_example.txt")
    x = workloads.f32_to_bf16_bits(np.array([[float(v) for v in r] for r in g["x"]], F32))
    w = workloads.f32_to_bf16_bits(np.array([[float(v) for v in r] for r in g["w"]], F32))
    # the fixture's decimal inputs are bf16 values: the bits must round-trip
    assert np.array_equal(f32(x), np.array([[float(v) for v in r] for r in g["x"]], F32))
    qx, dx = orc.quant_act(x)
    qw, dw = orc.quant_weight(w)
    assert np.array_equal(qx, np.array([[int(v, 16) for v in r] for r in g["qx"]], np.uint8))
    assert np.array_equal(qw, np.array([[int(v, 16) for v in r] for r in g["qw"]], np.uint8))
    assert np.array_equal(dx, np.array([float(v) for v in g["dx"][0]], F32))
    assert np.array_equal(dw, np.array([float(v) for v in g["dw"][0]], F32))


def test_amax_element_encodes_to_448(orc, cfg2):
    _, x, w = cfg2
    for mat, quant, axis in ((x, orc.quant_act, 1), (w.T.copy(), orc.quant_act, 1)):
        q, d = quant(mat)
        a = np.abs(f32(mat))
        nz = a.max(axis=axis) > 0
        idx = a.argmax(axis=axis)
        picked = q[np.arange(q.shape[0]), idx]
        assert np.all((picked[nz] & 0x7F) == 0x7E)
        assert np.all(d[~nz] == 1.0)


def test_scale_is_nearest_fp32_to_amax_over_448(orc):
    rng = np.random.default_rng(1)
    x = workloads.random_bf16(rng, 64, 200, sigma=1.0)
    x[5] = workloads.f32_to_bf16_bits(np.full(200, 3.0e-38, F32))   # tiny amax
    x[6] = workloads.f32_to_bf16_bits(np.full(200, 1.0e30, F32))    # huge amax
    _, d = orc.quant_act(x)
    for t in range(x.shape[0]):
        amax = np.abs(f32(x[t])).max()
        want = nearest_f32(Fraction(float(amax)) / 448)
        assert d[t] == want, t


def test_zero_row(orc, cfg2):
    _, x, _ = cfg2
    zero_rows = np.flatnonzero(np.all(f32(x) == 0, axis=1))
    assert zero_rows.size == 1
    q, d = orc.quant_act(x)
    assert d[zero_rows[0]] == 1.0
    assert np.all(q[zero_rows[0]] == 0)
    # a row of negative zeros keeps the sign bit
    q2, d2 = orc.quant_act(np.full((1, 16), 0x8000, np.uint16))
    assert d2[0] == 1.0 and np.all(q2 == 0x80)


@pytest.mark.parametrize("k", [-5, -1, 1, 4])
def test_power_of_two_equivariance(orc, cfg2, k):
    _, x, _ = cfg2
    xs = x[:8]
    scaled = workloads.f32_to_bf16_bits(f32(xs) * F32(2.0 ** k))
    assert np.array_equal(f32(scaled), f32(xs) * F32(2.0 ** k))     # exact
    q0, d0 = orc.quant_act(xs)
    q1, d1 = orc.quant_act(scaled)
    assert np.array_equal(q0, q1)
    nz = d0 != 1.0
    assert np.array_equal(d1[nz], d0[nz] * F32(2.0 ** k))


def test_negation_flips_sign_bit_only(orc, cfg2):
    _, x, _ = cfg2
    q0, d0 = orc.quant_act(x)
    q1, d1 = orc.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(d0, d1)
    assert np.array_equal(q1, q0 ^ np.uint8(0x80))


def test_error_bound(orc, cfg2):
    """|dec(q)*Delta - x| <= 2^-4 |x| where x/Delta is in E4M3's normal range,
    and <= 2^-10 Delta (+ fp32 slack) in the subnormal range."""
    _, x, _ = cfg2
    q, d = orc.quant_act(x)
    xv = f32(x).astype(np.float64)
    rec = orc.e4m3_decode(q) * d[:, None].astype(np.float64)
    ratio = np.abs(xv) / d[:, None]
    err = np.abs(rec - xv)
    normal = ratio >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xv[normal]))
    sub = ~normal
    assert np.all(err[sub] <= (2.0 ** -10 + 2.0 ** -20) * np.broadcast_to(d[:, None], xv.shape)[sub])


def test_shared_amax_reduces_to_per_tensor(orc):
    """Every row holding the same amax A: per-token codes and scales equal
    per-tensor FP8 with its single scale (the figure's top half)."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal((40, 300)).astype(F32) * 3
    v = np.clip(v, -9.5, 9.5)
    v[:, 7] = np.where(rng.random(40) < 0.5, 10.0, -10.0)   # |A| = 10 in every row
    x = workloads.f32_to_bf16_bits(v)
    q_tok, d_tok = orc.quant_act(x)
    q_ten, d_ten = orc.quant_tensor(x)
    assert np.all(d_tok == d_ten)
    assert np.array_equal(q_tok, q_ten)


def test_scale_one_equals_direct_torch_cast(orc):
    """amax = 448 gives Delta = 1, so every code is the plain cast of the bf16
    value -- compare with PyTorch's float8_e4m3fn cast (ties included: bf16
    carries 7 mantissa bits, E4M3 keeps 3)."""
    b = np.arange(1 << 16, dtype=np.uint32)
    vals = (b << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    n = 512
    rows = -(-vals.size // (n - 1))
    pad = np.zeros(rows * (n - 1), F32)
    pad[:vals.size] = vals
    m = np.concatenate([np.full((rows, 1), 448.0, F32), pad.reshape(rows, n - 1)], axis=1)
    x = workloads.f32_to_bf16_bits(m)
    q, d = orc.quant_act(x)
    assert np.all(d == 1.0)
    want = torch.from_numpy(m.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_weight_quant_is_act_quant_of_transpose(orc):
    """One scale per output column o of W [Ci x Co]: quantizing W must equal
    quantizing the rows of W^T (catches a per-input-channel slip)."""
    rng = np.random.default_rng(9)
    w = workloads.random_bf16(rng, 96, 80, sigma=0.02)
    w[:, 3] = 0
    qw, dw = orc.quant_weight(w)
    qt, dt = orc.quant_act(np.ascontiguousarray(w.T))
    assert dw.shape == (80,)
    assert np.array_equal(dw, dt)
    assert np.array_equal(qw, qt.T)


# -- static per-tensor (the "standard FP8" comparator with a given scale) -----
def test_static_with_measured_scale_is_per_tensor(orc):
    """Given the scale the per-tensor quantizer measures, static quantization
    reproduces its codes."""
    rng = np.random.default_rng(21)
    x = workloads.random_bf16(rng, 33, 272, 1.5)
    q_ten, d_ten = orc.quant_tensor(x)
    assert np.array_equal(orc.quant_static(x, d_ten), q_ten)


def test_static_scale_one_is_torch_cast(orc):
    """s = 1: every code is the plain cast of the bf16 value (within +-448,
    where PyTorch's float8_e4m3fn cast is defined without saturation)."""
    b = np.arange(1 << 16, dtype=np.uint32)
    vals = (b << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    n = 1024
    pad = np.zeros(-(-vals.size // n) * n, F32)
    pad[:vals.size] = vals
    m = pad.reshape(-1, n)
    x = workloads.f32_to_bf16_bits(m)
    want = torch.from_numpy(m.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.quant_static(x, 1.0), want)


def test_static_saturates_beyond_range(orc):
    """A static scale can be too small for the data: quotients beyond 448
    (464 included, the tie between 448 and the next binade) saturate to the
    largest finite code, sign kept; NaN codes never appear."""
    v = np.array([[449.0, 464.0, 465.0, 1e6, -449.0, -464.0, -1e6, 3.0e38]], F32)
    q = orc.quant_static(workloads.f32_to_bf16_bits(v), 1.0)
    assert q.tolist() == [[0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE, 0x7E]]
    q2 = orc.quant_static(workloads.f32_to_bf16_bits(np.array([[8.0, -8.0, -0.5]], F32)), 2.0 ** -6)
    assert q2.tolist() == [[0x7E, 0xFE, 0xE0]]            # -0.5 / 2^-6 = -32 is in range


def test_per_tensor_amax_spans_every_row_and_column(orc):
    """Per-tensor FP8 ([PTPC] §Understanding the figure, one scalar scale for
    the whole tensor) on a matrix whose rows all have different maxima, the
    largest in the last row and last column: the scale is the fp32 nearest to
    that element's magnitude / 448 (exact rationals), and every code is the
    brute-force nearest E4M3 (ties to even) of the IEEE fp32 quotient.  An
    amax that reads only some rows or columns gives another scale and fails."""
    from test_oracle_codec import brute_force_encode
    rng = np.random.default_rng(9)
    R, C = 37, 48
    v = rng.standard_normal((R, C)).astype(F32)
    v *= (1.0 + np.arange(R, dtype=F32)[:, None] / 4)          # row maxima differ
    v[R - 1, C - 1] = -300.5                                    # the tensor's largest
    x = workloads.f32_to_bf16_bits(v)
    xf = f32(x)
    assert np.abs(xf).argmax() == R * C - 1
    q, d = orc.quant_tensor(x)
    want_d = nearest_f32(Fraction(float(np.abs(xf).max())) / 448)
    assert d == want_d
    assert q[R - 1, C - 1] == 0xFE
    assert np.array_equal(q, brute_force_encode((xf / np.float32(d)).astype(F32)))
