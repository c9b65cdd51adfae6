"""ptpc_gemm_noalloc (the entry point for callers that cannot allocate)
against ptpc_gemm_ws with a caller workspace, through the C ABI.

Both run the same split-K kernels in the same summation order, so the
outputs must be bit-identical; four calls in a row, each on a smaller
split than the one before (the scratch keeps the previous call's partial
sums) -- the first fills the whole scratch, the second joins two K ranges
inside the GEMM kernel through per-tile records in the scratch -- and a
shape that does not split (then both equal ptpc_gemm).  The first three
outputs are also held to the accuracy bar against the oracle on sampled
outputs, the last one on its whole output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (bits_to_dev, check_close, dev_to_bits, nan_filled, no_nan,
                         oracle_sampled_ref, sample_indices)

pytestmark = pytest.mark.gpu


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


def inputs(sg, T, Ci, Co, seed):
    rng = np.random.default_rng(seed)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, ::53] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, ::53]) * np.float32(40))
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    return x, w, qx, dx, pw


def both(sg, qx, dx, pw, T, Co):
    a = sg.gemm_noalloc(qx, dx, pw, out=nan_filled(T, Co))
    b = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co))
    torch.cuda.synchronize()
    no_nan(a, "noalloc")
    return dev_to_bits(a), dev_to_bits(b)


def test_noalloc_matches_workspace_form(sg):
    # 1: the 70B down projection at 256 tokens: 256x256 tiles, K split 8
    #    ways, 64 MiB of partial sums (the whole scratch)
    shape, x, w = workloads.make("70b_down", T=256)
    T, Ci, Co = shape.T, shape.Ci, shape.Co
    need0 = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need0 == sg.NOALLOC_SCRATCH_BYTES
    note(f"noalloc call 1: T={T} Ci={Ci} Co={Co} scratch {need0} bytes")
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    a, b = both(sg, qx, dx, pw, T, Co)
    assert np.array_equal(a, b), "noalloc != workspace form (call 1)"
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    rows, cols = sample_indices(T, Co, 2000, seed=4)
    check_close(a[rows, cols], oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols),
                "noalloc 70b down T=256 (sampled)")
    del qx, dx, pw, x, w, qw_o
    # 2: two K ranges over 256x256 tiles joined inside the GEMM kernel
    #    (8 x 11 tiles, ragged rows, columns and K tail): per-tile slots
    #    and records in the scratch, the records cleared by the call
    T, Ci, Co = 1793, 16400, 2576
    need_fix = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need_fix == 88 * (4 * 256 * 256 + 16) and need_fix < need0
    note(f"noalloc call 2: T={T} Ci={Ci} Co={Co} scratch {need_fix} bytes")
    x, w, qx, dx, pw = inputs(sg, T, Ci, Co, seed=6)
    a, b = both(sg, qx, dx, pw, T, Co)
    assert np.array_equal(a, b), "noalloc != workspace form (call 2)"
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    rows, cols = sample_indices(T, Co, 2000, seed=6)
    check_close(a[rows, cols], oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols),
                "noalloc two-range fix-up (sampled)")
    del qx, dx, pw, x, w, qw_o
    # 3: the 70B QKV projection at 128 tokens: 128x128 tiles, K split 3
    #    ways, 15.7 MB of partial sums
    shape, x, w = workloads.make("70b_sweep", T=128, layer="qkv")
    T, Ci, Co = shape.T, shape.Ci, shape.Co
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert 0 < need < need_fix
    note(f"noalloc call 3: T={T} Ci={Ci} Co={Co} scratch {need} bytes")
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    a, b = both(sg, qx, dx, pw, T, Co)
    assert np.array_equal(a, b), "noalloc != workspace form (call 3)"
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    rows, cols = sample_indices(T, Co, 2000, seed=5)
    check_close(a[rows, cols], oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols),
                "noalloc 70b qkv T=128 (sampled)")
    del qx, dx, pw
    # 4: a smaller split (4 K ranges, ragged rows, columns and K tail) right
    #    after, over the scratch the previous calls left behind
    T, Ci, Co = 150, 4112, 256
    assert 0 < sg.gemm_workspace_bytes(T, Ci, Co) < need
    note(f"noalloc call 4: T={T} Ci={Ci} Co={Co}")
    x, w, qx, dx, pw = inputs(sg, T, Ci, Co, seed=2)
    a, b = both(sg, qx, dx, pw, T, Co)
    assert np.array_equal(a, b), "noalloc != workspace form (call 4)"
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    check_close(a, oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o),
                "noalloc ragged split")


def test_noalloc_without_split_is_gemm(sg):
    T, Ci, Co = 300, 1040, 784
    assert sg.gemm_workspace_bytes(T, Ci, Co) == 0
    note(f"noalloc no split: T={T} Ci={Ci} Co={Co}")
    _, _, qx, dx, pw = inputs(sg, T, Ci, Co, seed=3)
    a = dev_to_bits(sg.gemm_noalloc(qx, dx, pw))
    b = dev_to_bits(sg.gemm(qx, dx, pw))
    assert np.array_equal(a, b)
