"""The Python binding refuses mismatched buffers before calling the library
(CPU only).

The kernels trust the extents they are given, so an output, code buffer,
scale vector or workspace of the wrong size, type or place would be read or
written out of bounds on the GPU.  Here the library's compute entry points
are replaced by a stand-in that fails the test if it is ever called, and the
device check is relaxed so that CPU tensors stand in for GPU ones; every
mismatch must raise before any call.
"""
import pytest
import torch

import scaled_gemm_amd as sg


class NoCompute:
    """The real library for size and kernel queries; any compute call fails."""
    QUERIES = {"ptpc_weight_packed_bytes", "ptpc_gemm_workspace_bytes",
               "ptpc_gemm_unfused_workspace_bytes", "ptpc_gemm_unfused_bf16_workspace_bytes",
               "ptpc_gemm_kernel", "ptpc_quant_act_kernel", "ptpc_gemm_ws_splits",
               "ptpc_status_string"}

    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in self.QUERIES:
            return getattr(self.real, name)

        def call(*a):
            raise AssertionError(f"{name} was called with a mismatched argument")
        return call


@pytest.fixture
def cpu_binding(monkeypatch):
    real = sg.lib()
    monkeypatch.setattr(sg, "_lib", NoCompute(real))
    monkeypatch.setattr(sg, "_on_gpu", lambda t, name: None)
    yield


T, Ci, Co = 6, 64, 48


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def weight(per_tensor=False, Ci=Ci, Co=Co, dw_len=None):
    n = sg.packed_bytes(Ci, Co)
    return sg.PackedWeight(u8(n), f32(dw_len if dw_len is not None else (1 if per_tensor else Co)),
                           Ci, Co, per_tensor=per_tensor)


def raises(fn, match):
    with pytest.raises((ValueError, TypeError), match=match):
        fn()


def test_quantizers(cpu_binding):
    x = bf16(T, Ci)
    raises(lambda: sg.quant_act(x, qx=u8(T, Ci - 16)), "qx: expected shape")
    raises(lambda: sg.quant_act(x, qx=u8(T + 1, Ci)), "qx: expected shape")
    raises(lambda: sg.quant_act(x, dx=f32(T - 1)), "dx: expected 6 elements")
    raises(lambda: sg.quant_act(x, dx=torch.zeros(T, dtype=torch.float64)), "dx: expected")
    raises(lambda: sg.quant_act(x, dx=f32(2 * T)[::2]), "dx: expected a contiguous")
    raises(lambda: sg.quant_act(x.float()), "x: expected torch.bfloat16")
    w = bf16(Ci, Co)
    raises(lambda: sg.quant_weight(w, out=weight(Co=Co + 16)), "PackedWeight is")
    raises(lambda: sg.quant_weight(w, out=weight(dw_len=Co - 1)), "out.dw")
    small = sg.PackedWeight(u8(10), f32(Co), Ci, Co)
    raises(lambda: sg.quant_weight(w, out=small), "out.data")
    raises(lambda: sg.quant_weight(w, out=weight(per_tensor=True)), "per-tensor weight")
    raises(lambda: sg.unpack_weight(small), "pw.data")
    raises(lambda: sg.tensor_scale(x, d=f32(2)), "d: expected 1 elements")
    raises(lambda: sg.quant_act_static(x, f32(1), qx=u8(T, Ci + 16)), "qx: expected shape")
    raises(lambda: sg.quant_act_static(x, f32(0)), "d: expected 1 elements")
    raises(lambda: sg.quant_weight_static(w, f32(1), out=weight()), "per-channel weight")


@pytest.mark.parametrize("call", ["gemm", "gemm_ws", "gemm_unfused", "gemm_unfused_bf16"])
def test_per_token_gemms(cpu_binding, call):
    fn = getattr(sg, call)
    qx, dx, pw = u8(T, Ci), f32(T), weight()
    raises(lambda: fn(qx, dx, pw, out=bf16(T, Co - 16)), "out: expected shape")
    raises(lambda: fn(qx, dx, pw, out=bf16(T + 1, Co)), "out: expected shape")
    raises(lambda: fn(qx, dx, pw, out=torch.zeros((T, Co), dtype=torch.float16)), "out: expected")
    raises(lambda: fn(qx, f32(T - 1), pw), "dx: expected 6 elements")
    raises(lambda: fn(qx, torch.zeros(T, dtype=torch.float64), pw), "dx: expected")
    raises(lambda: fn(u8(T, Ci + 16), dx, pw), "has Ci=")
    raises(lambda: fn(qx, dx, weight(dw_len=1)), "pw.dw")
    raises(lambda: fn(qx, dx, weight(per_tensor=True)), "per-tensor weight")
    raises(lambda: fn(qx, dx, sg.PackedWeight(u8(100), f32(Co), Ci, Co)), "pw.data")


def test_workspaces(cpu_binding):
    qx, dx, pw = u8(T, Ci), f32(T), weight()
    raises(lambda: sg.gemm_unfused(qx, dx, pw, workspace=f32(T, Co - 1)), "at least")
    raises(lambda: sg.gemm_unfused(qx, dx, pw, workspace=bf16(T, Co)), "workspace: expected")
    raises(lambda: sg.gemm_unfused_bf16(qx, dx, pw, workspace=bf16(T, Co - 1)), "at least")
    raises(lambda: sg.gemm_unfused_bf16(qx, dx, pw, workspace=f32(T, Co)), "workspace: expected")
    # a shape that splits K needs its full workspace
    Tw, Ciw, Cow = 128, 8192, 10240
    need = sg.gemm_workspace_bytes(Tw, Ciw, Cow)
    assert need > 0
    raises(lambda: sg.gemm_ws(u8(Tw, Ciw), f32(Tw), weight(Ci=Ciw, Co=Cow),
                              workspace=u8(need - 16)), "workspace: expected at least")


def test_per_tensor_gemm(cpu_binding):
    qx = u8(T, Ci)
    raises(lambda: sg.gemm_tensor(qx, f32(1), weight()), "per-channel weight")
    raises(lambda: sg.gemm_tensor(qx, f32(2), weight(per_tensor=True)), "dx: expected 1")
    raises(lambda: sg.gemm_tensor(qx, f32(1), weight(per_tensor=True), out=bf16(T, 16)),
           "out: expected shape")


def test_cpu_tensors_are_refused():
    """Without the relaxed device check, host tensors never reach the library."""
    sg.lib()
    with pytest.raises(ValueError, match="on the GPU"):
        sg.quant_act(bf16(T, Ci))
    with pytest.raises(ValueError, match="on the GPU"):
        sg.gemm(u8(T, Ci), f32(T), weight())
