"""Seeded random shapes through every entry point of the path, whole outputs
against the oracle, through the C ABI.

The fixed-shape parity cases target each kernel and tile on purpose; these
draw token counts, K and output widths at random (ragged everywhere:
multiples of 16 that are rarely multiples of a tile) from every token range
the kernel choice distinguishes, plus a few wide layers, and check on each:
activation codes and scales and weight codes and scales bit-exact, the fused
GEMM's whole output within the bar (every element written: the buffer starts
as NaN), the two-step form equal to the fused one bit for bit, and the
workspace form within the bar on its whole output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bits_to_dev, check_close, dev_to_bits, nan_filled, no_nan

pytestmark = pytest.mark.gpu

# (lowest T, highest T, count) per token range of the kernel choice.
T_RANGES = [(1, 8, 15), (9, 32, 15), (33, 64, 15), (65, 128, 16), (129, 255, 16), (256, 700, 17)]


def shapes():
    rng = np.random.default_rng(2024)
    out = []
    for lo, hi, n in T_RANGES:
        for _ in range(n):
            T = int(rng.integers(lo, hi + 1))
            Ci = 16 * int(rng.integers(1, 130))          # 16 .. 2064
            Co = 16 * int(rng.integers(1, 130))
            out.append((T, Ci, Co))
    # wide layers (kernels chosen only for many output columns), short K
    for T in (40, 100, 200, 300):
        out.append((T, 16 * int(rng.integers(4, 20)), 16 * int(rng.integers(2100, 3200))))
    # long K with few output tiles: the workspace form splits K
    for lo, hi in ((65, 128), (129, 255), (256, 400), (256, 400)):
        out.append((int(rng.integers(lo, hi + 1)), 16 * int(rng.integers(1024, 1250)),
                    16 * int(rng.integers(16, 64))))
    return out


SHAPES = shapes()


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_gemm_amd
    scaled_gemm_amd.lib()
    return scaled_gemm_amd


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("T,Ci,Co", SHAPES)
def test_random_shape(sg, T, Ci, Co):
    note(f"random shape T={T} Ci={Ci} Co={Co}: {sg.gemm_kernel(T, Ci, Co)}, "
         f"{sg.gemm_ws_splits(T, Ci, Co)} K range(s)")
    rng = np.random.default_rng([T, Ci, Co])
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    hot = rng.choice(Ci, size=max(1, Ci // 50), replace=False)
    x[:, hot] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, hot]) * np.float32(40))
    if T > 3:
        x[T // 2] = 0
    w = workloads.random_bf16(rng, Ci, Co, 0.02)

    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    assert np.array_equal(qx.cpu().numpy(), qx_o), "activation codes"
    assert np.array_equal(dx.cpu().numpy(), dx_o), "activation scales"
    assert np.array_equal(pw.dw.cpu().numpy(), dw_o), "weight scales"
    assert np.array_equal(sg.unpack_weight(pw).cpu().numpy(), qw_o), "weight codes"

    ref = oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o)
    fused = sg.gemm(qx, dx, pw, out=nan_filled(T, Co))
    no_nan(fused, "fused")
    a = dev_to_bits(fused)
    check_close(a, ref, f"random T={T} Ci={Ci} Co={Co} fused")
    b = dev_to_bits(sg.gemm_unfused(qx, dx, pw))
    assert np.array_equal(a, b), "fused and two-step differ"
    ws = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co))
    no_nan(ws, "workspace form")
    check_close(dev_to_bits(ws), ref, f"random T={T} Ci={Ci} Co={Co} workspace form")
