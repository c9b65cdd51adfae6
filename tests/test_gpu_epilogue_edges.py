"""Bit-exact check of the GEMM epilogue on edge values, every kernel family.

The epilogue turns an fp32 accumulator into out = bf16((acc * dx[t]) * dw[o])
(vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm", §Understanding
the figure: the token scale and the channel scale applied to the FP8 product),
two fp32 products, then rounding to nearest, ties to even.  Here the operands
are chosen so that every accumulator is exact in fp32 whatever the summation
order (values m * 2^e with 3-bit m and e in {-1, 0, 1}: products on a 2^-8
grid, sums below 2^16), which makes each output one fixed bf16 pattern; the
scale vectors are then chosen to land on the edges of that rounding: exact
ties (both directions of ties-to-even), subnormal results, overflow to
infinity and values next to the largest finite bf16.  Expected values come
from the oracle's exact sums, numpy's IEEE fp32 products and a rounding
written from the definition (nearest of the two neighbouring bf16 values by
exact distance, ties to the even one).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity_shapes as ps
import workloads
from gpu_helpers import bits_to_dev, dev_to_bits

sg = None


@pytest.fixture(scope="module")
def gpu_lib():
    global sg
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_gemm_amd
    sg = scaled_gemm_amd
    sg.lib()
    yield


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_nearest_even(f):
    """fp32 (finite or infinite, no NaN) -> bf16 bits: the nearer of the two
    bf16 values that bracket |f|, the one with an even last bit on a tie, and
    a magnitude past the largest finite value's half step becomes infinity."""
    f = np.asarray(f, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    sign = (u >> 16) & 0x8000
    mag = u & 0x7FFFFFFF
    lo = mag & 0xFFFF0000                                   # bracket below (or equal)
    hi = lo + 0x10000                                       # next bf16 above
    x = mag.astype(np.uint32).view(np.float32).astype(np.float64)
    lo_v = lo.astype(np.uint32).view(np.float32).astype(np.float64)
    hi_v = np.where(hi >= 0x7F800000, 2.0 ** 128,
                    np.minimum(hi, 0x7F7F0000).astype(np.uint32).view(np.float32).astype(np.float64))
    with np.errstate(invalid="ignore"):                    # inf - inf on infinite inputs
        d_lo, d_hi = x - lo_v, hi_v - x
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (((lo >> 16) & 1) == 1))
    res = np.where(up, hi >> 16, lo >> 16)
    res = np.where(mag >= 0x7F800000, 0x7F80, res)          # infinity stays infinity
    return (res | sign).astype(np.uint16)


def test_nearest_even_reference_pins():
    """The test's own rounding on hand-picked values (CPU only): exact,
    both tie directions, just above a tie, subnormal (below half the
    smallest, exact, tie), the largest finite fp32 (rounds to infinity), the
    largest finite bf16, infinities, zero."""
    one_plus = lambda k: np.float32(1 + k * 2.0 ** -8)
    vals = np.array([1.0, one_plus(1), one_plus(3), np.float32(1 + 2.0 ** -8 + 2.0 ** -20),
                     -1.5, 2.0 ** -149, 2.0 ** -133, 3 * 2.0 ** -134,
                     np.finfo(np.float32).max, np.uint32(0x7F7F0000).view(np.float32),
                     np.inf, -np.inf, 0.0], np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBFC0, 0x0000, 0x0001, 0x0002,
            0x7F80, 0x7F7F, 0x7F80, 0xFF80, 0x0000]
    assert bf16_nearest_even(vals).tolist() == want


def _values(rng, shape):
    """Random m * 2^e, m in {1, 1.125, ..., 1.875}, e in {-1, 0, 1}, either
    sign, a quarter of them zero; all exact in E4M3 and bf16."""
    m = 1 + rng.integers(0, 8, shape) / 8.0
    e = rng.integers(-1, 2, shape).astype(np.float64)
    s = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    v = s * m * 2.0 ** e
    v[rng.random(shape) < 0.25] = 0.0
    return v


def edge_case(T, Ci, Co, seed):
    """Inputs whose quantization is exact (scales 1: a 448 in a K position the
    other operand leaves zero) and the edge-value scale vectors."""
    rng = np.random.default_rng(seed)
    x = _values(rng, (T, Ci))
    w = _values(rng, (Ci, Co))
    x[:, 0] = 0.0
    x[:, 1] = 448.0                       # row amax -> dx = 1, meets w[1, :] = 0
    w[0, :] = 448.0                       # column amax -> dw = 1, meets x[:, 0] = 0
    w[1, :] = 0.0
    cat_t = np.arange(T) % 6
    for t in np.nonzero(cat_t == 1)[0]:   # one nonzero product per output: acc = w[k, o]
        k = 2 + int(t) % (Ci - 2)
        x[t, 2:] = 0.0
        x[t, k] = 1.0
    x[cat_t == 5, 2:] = 0.0               # zero rows
    dx = np.empty(T, np.float32)
    dx[cat_t == 0] = rng.uniform(0.5, 2.0, int(np.sum(cat_t == 0))).astype(np.float32)
    dx[cat_t == 1] = 1.0
    dx[cat_t == 2] = 2.0 ** -120          # subnormal results with dw = 2^-12
    dx[cat_t == 3] = 2.0 ** 100           # overflow with dw = 2^30
    dx[cat_t == 4] = 2.0 ** 120           # next to the largest finite with dw = 2^7
    dx[cat_t == 5] = 3.0
    cat_o = np.arange(Co) % 6
    dw = np.empty(Co, np.float32)
    dw[cat_o == 0] = rng.uniform(0.5, 2.0, int(np.sum(cat_o == 0))).astype(np.float32)
    dw[cat_o == 1] = 1 + 2.0 ** -8        # acc = 1: tie, rounds down to even
    dw[cat_o == 2] = 2.0 ** -12
    dw[cat_o == 3] = 2.0 ** 30
    dw[cat_o == 4] = 2.0 ** 7
    dw[cat_o == 5] = 1 + 3 * 2.0 ** -8    # acc = 1: tie, rounds up to even
    return (workloads.f32_to_bf16_bits(x.astype(np.float32)),
            workloads.f32_to_bf16_bits(w.astype(np.float32)), dx, dw)


def expected(x_bits, w_bits, dx, dw):
    qx, sx = oracle.quant_act(x_bits)
    qw, sw = oracle.quant_weight(w_bits)
    assert np.all(sx == 1) and np.all(sw == 1)
    acc = oracle.gemm_exact(qx, qw)
    acc32 = acc.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), acc), "accumulators not exact in fp32"
    with np.errstate(over="ignore", under="ignore"):
        out32 = (acc32 * dx[:, None]).astype(np.float32) * dw[None, :]
        ws_bf = bf16_nearest_even(acc32)
        ws32 = (ws_bf.astype(np.uint32) << 16).view(np.float32)
        out_bf32 = (ws32 * dx[:, None]).astype(np.float32) * dw[None, :]
    ties = int(np.sum((out32.view(np.uint32) & 0xFFFF) == 0x8000))
    assert ties > 0, "no exact ties among the outputs"
    return qx, qw, bf16_nearest_even(out32), ws_bf, bf16_nearest_even(out_bf32)


def same_bits(got, want, what):
    """Bit equality, with +0 and -0 taken as equal (the sign of an exact zero
    sum is not part of the method)."""
    zero = ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    bad = np.argwhere((got != want) & ~zero)
    assert bad.size == 0, (f"{what}: {len(bad)} outputs differ, first "
                           f"{[(int(t), int(o), hex(got[t, o]), hex(want[t, o])) for t, o in bad[:4]]}")


# The shape picks the kernel family (see parity_shapes.EPILOGUE_CASES).
@pytest.mark.gpu
@pytest.mark.parametrize("T,Ci,Co", ps.EPILOGUE_CASES)
def test_epilogue_edge_values(gpu_lib, T, Ci, Co):
    note(f"epilogue edges T={T} Ci={Ci} Co={Co}")
    x, w, dx, dw = edge_case(T, Ci, Co, seed=T)
    qx_o, qw_o, want, ws_want, want_bf = expected(x, w, dx, dw)
    qx, sx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    assert np.array_equal(qx.cpu().numpy(), qx_o)
    assert np.array_equal(sg.unpack_weight(pw).cpu().numpy(), qw_o)
    dxd = torch.from_numpy(dx).cuda()
    pwd = sg.PackedWeight(pw.data, torch.from_numpy(dw).cuda(), Ci, Co)
    subnormal = ((want & 0x7F80) == 0) & ((want & 0x7F) != 0)
    assert np.sum(want == 0x7F80) > 0 and np.sum(subnormal) > 0
    same_bits(dev_to_bits(sg.gemm(qx, dxd, pwd)), want, "fused")
    same_bits(dev_to_bits(sg.gemm_ws(qx, dxd, pwd)), want, "workspace form")
    same_bits(dev_to_bits(sg.gemm_unfused(qx, dxd, pwd)), want, "two-step fp32")
    ws3 = torch.empty((T, Co), dtype=torch.bfloat16, device="cuda")
    out3 = sg.gemm_unfused_bf16(qx, dxd, pwd, workspace=ws3)
    torch.cuda.synchronize()
    same_bits(dev_to_bits(ws3), ws_want, "two-step bf16 intermediate")
    same_bits(dev_to_bits(out3), want_bf, "two-step bf16")
