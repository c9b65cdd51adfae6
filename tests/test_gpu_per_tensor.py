"""GPU parity of the per-tensor ("standard FP8") comparator against the oracle.

Scales and codes bit-identical to the oracle's per-tensor and static
quantizers; GEMM outputs within the bf16 bar of the exact-sum reference, and
bit-identical to the per-token / per-channel GEMM fed the same scalar scale
in every row and column (the same epilogue arithmetic).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity_shapes as ps
import workloads
from gpu_helpers import (bits_to_dev, check_close, dev_to_bits, oracle_sampled_ref,
                         packed_byte_index, sample_indices)

pytestmark = pytest.mark.gpu

sg = None


@pytest.fixture(scope="module", autouse=True)
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


def f32(d):
    return float(np.float32(d))


def per_tensor_path(x_bits, w_bits):
    x, w = bits_to_dev(x_bits), bits_to_dev(w_bits)
    sx = sg.tensor_scale(x)
    sw = sg.tensor_scale(w)
    qx = sg.quant_act_static(x, sx)
    pw = sg.quant_weight_static(w, sw)
    out = sg.gemm_tensor(qx, sx, pw)
    # the per-token GEMM fed the scalar scales in every row / column
    pw_b = sg.PackedWeight(pw.data, sw.expand(pw.Co).contiguous(), pw.Ci, pw.Co)
    out_b = sg.gemm(qx, sx.expand(qx.shape[0]).contiguous(), pw_b)
    qw = sg.unpack_weight(pw)
    torch.cuda.synchronize()
    return dict(sx=sx.cpu().numpy()[0], sw=sw.cpu().numpy()[0], qx=qx.cpu().numpy(),
                qw=qw.cpu().numpy(), packed=pw.data.cpu().numpy(), out=dev_to_bits(out),
                out_b=dev_to_bits(out_b))


def check_per_tensor_quant(g, x_bits, w_bits, what):
    qx_o, sx_o = oracle.quant_tensor(x_bits)
    qw_o, sw_o = oracle.quant_tensor(w_bits)
    assert g["sx"] == sx_o and g["sw"] == sw_o, f"{what}: scales differ"
    assert np.array_equal(g["qx"], qx_o), f"{what}: activation codes differ"
    assert np.array_equal(g["qw"], qw_o), f"{what}: weight codes differ"
    Ci, Co = w_bits.shape
    if Ci * Co <= (1 << 26):
        idx = packed_byte_index(Ci, Co)
        assert np.array_equal(g["packed"][idx[:Ci]], qw_o), f"{what}: packed layout"
        assert np.all(g["packed"][idx[Ci:]] == 0), f"{what}: K padding not zero"
    return qx_o, sx_o, qw_o, sw_o


CASES = ps.PER_TENSOR_CASES


@pytest.mark.parametrize("name,T,Ci,Co", CASES)
def test_per_tensor_full(name, T, Ci, Co):
    note(f"per-tensor {name} T={T} Ci={Ci} Co={Co}")
    if name == "ragged":
        rng = np.random.default_rng(T * 11 + Ci)
        x = workloads.random_bf16(rng, T, Ci, 1.0)
        x[:, :: max(1, Ci // 5)] = workloads.f32_to_bf16_bits(
            workloads.bf16_bits_to_f32(x[:, :: max(1, Ci // 5)]) * np.float32(40))
        w = workloads.random_bf16(rng, Ci, Co, 0.02)
    else:
        _, x, w = workloads.make(name)
    g = per_tensor_path(x, w)
    qx, sx, qw, sw = check_per_tensor_quant(g, x, w, name)
    acc = oracle.gemm_exact(qx, qw)
    ref = oracle.apply_scales(acc, np.full(T, sx, np.float32), np.full(Co, sw, np.float32))
    check_close(g["out"], ref, f"{name} per-tensor")
    assert np.array_equal(g["out"], g["out_b"]), "per-tensor GEMM != broadcast per-token GEMM"


def test_per_tensor_70b_down_sampled():
    note("per-tensor 70b_down (sampled GEMM)")
    shape, x, w = workloads.make("70b_down")
    g = per_tensor_path(x, w)
    qx, sx, qw, sw = check_per_tensor_quant(g, x, w, "70b_down")
    T, Co = shape.T, shape.Co
    rows, cols = sample_indices(T, Co, 3000, seed=5)
    ref = oracle_sampled_ref(qx, np.full(T, sx, np.float32), qw, np.full(Co, sw, np.float32),
                             rows, cols)
    check_close(g["out"].reshape(T, Co)[rows, cols], ref, "70b_down per-tensor (sampled)")
    assert np.array_equal(g["out"], g["out_b"])


def test_static_scales_given():
    """Static (given) scales, including ones too small for the data: codes
    equal the oracle's static quantizer, saturation included."""
    rng = np.random.default_rng(17)
    x = workloads.random_bf16(rng, 70, 528, 3.0)
    w = workloads.random_bf16(rng, 528, 208, 0.05)
    for s in (1.0, 2.0 ** -6, 0.0123, 37.5, 1e-30):
        note(f"static scale {s}")
        d = torch.tensor([s], dtype=torch.float32, device="cuda")
        qx = sg.quant_act_static(bits_to_dev(x), d).cpu().numpy()
        assert np.array_equal(qx, oracle.quant_static(x, f32(s))), f"activation codes, s={s}"
        pw = sg.quant_weight_static(bits_to_dev(w), d)
        assert np.array_equal(sg.unpack_weight(pw).cpu().numpy(), oracle.quant_static(w, f32(s)))


def test_tensor_scale_edges():
    """All-zero and empty matrices get scale 1; a single huge or subnormal
    value sets the scale exactly as the oracle's; pitched input."""
    z = torch.zeros((33, 64), dtype=torch.bfloat16, device="cuda")
    assert sg.tensor_scale(z).item() == 1.0
    e = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    assert sg.tensor_scale(e).item() == 1.0
    for bits in (0x0001, 0x7F7F, 0xFF7F, 0x43E0, 0x8080):
        m = np.zeros((37, 96), np.uint16)
        m[36, 95] = bits
        _, s_o = oracle.quant_tensor(m)
        assert sg.tensor_scale(bits_to_dev(m)).item() == float(s_o), hex(bits)
    rng = np.random.default_rng(4)
    wide = workloads.random_bf16(rng, 50, 160, 1.0)
    v = bits_to_dev(wide)[:, :144]
    _, s_o = oracle.quant_tensor(np.ascontiguousarray(wide[:, :144]))
    assert sg.tensor_scale(v).item() == float(s_o)
