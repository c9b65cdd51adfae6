"""The LDS-poison debug build (libptpc_lds_poison.so) against the release
build, bit for bit, through the C ABI.

In the debug build every pipelined GEMM kernel overwrites each LDS region
with E4M3 NaN bytes right before it issues the fills that refill it.  The
kernels run without a fence on their LDS-DMA fills and, in the K-split
kernel, without any barrier in the K loop; if a wave read a region after
another wave's refill had been issued, or before its own fill had landed,
it would read NaN and its outputs would be NaN, whatever the data.  Equal
outputs from both builds on a shape per pipelined kernel (fused, two-step and
split-K forms) are the evidence that no such read happens.
"""
import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

# One shape per pipelined kernel the tile rule can pick, with K remainders
# and ragged edges; (T, Ci, Co).
SHAPES = [
    (4096, 1648, 4096), (1536, 592, 8192), (1024, 880, 10240), (1024, 752, 14336),
    (256, 1040, 40944), (1024, 28672, 8192), (512, 16400, 1024), (100, 528, 1040),
    (120, 3344, 1040), (200, 144, 1040), (130, 272, 8208), (48, 272, 32784),
    (20, 144, 32784), (200, 272, 36864), (200, 272, 10240), (100, 272, 50192),
]
PIPELINED = {
    "gemm16_kernel<256,256,2,2>", "gemm16_kernel<192,256,2,2>", "gemm16_kernel<256,224,4,1>",
    "gemm16_kernel<256,160,2,2>", "gemm16_kernel<128,256,2,2>",
    "gemm16_kernel<128,128,2,2>", "gemm16_kernel<128,224,2,2>", "gemm16s_kernel",
    "gemm_kernel<64,64,2,2,4>",
    "gemm_kernel<64,128,2,2,4>", "gemm_kernel<128,128,2,2,4>", "gemm_kernel<32,64,1,2,4>",
}
# The split-K forms of ptpc_gemm_ws: 128x128 tiles of the 32x32x64 kernel
# (4 K ranges, then the reduction pass), 256x256 tiles (8 ranges, reduction
# pass), and two ranges of 256x256 tiles joined inside the kernel.
SPLIT_K = [(200, 4112, 400, 4), (300, 12304, 528, 8), (1024, 16400, 8192, 2)]


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_gemm_amd as sg
    from scaled_gemm_amd import build
    sg.lib()
    assert os.path.exists(build.POISON_LIB), "build the LDS-poison variant first"
    P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L = ctypes.CDLL(build.POISON_LIB)
    for f in ("ptpc_gemm",):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [P, I, P, P, P, I, I, I, P, I, P]
    L.ptpc_gemm_unfused.restype = ctypes.c_int
    L.ptpc_gemm_unfused.argtypes = [P, I, P, P, P, I, I, I, P, I, P, P]
    L.ptpc_gemm_ws.restype = ctypes.c_int
    L.ptpc_gemm_ws.argtypes = [P, I, P, P, P, I, I, I, P, I, P, S, P]
    return sg, L


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def operands(sg, T, Ci, Co, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((T, Ci), generator=g, device="cuda").to(torch.bfloat16)
    x[:, ::37] *= 30
    w = (0.02 * torch.randn((Ci, Co), generator=g, device="cuda")).to(torch.bfloat16)
    qx, dx = sg.quant_act(x)
    return qx, dx, sg.quant_weight(w)


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def run_poison(L, fn, qx, dx, pw, out, *extra):
    T, Ci = qx.shape
    st = getattr(L, fn)(p(qx), Ci, p(dx), p(pw.data), p(pw.dw), T, Ci, pw.Co, p(out), pw.Co,
                        *extra, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"{fn} -> {st}"


def test_shapes_cover_every_pipelined_kernel(libs):
    sg, _ = libs
    assert {sg.gemm_kernel(*s) for s in SHAPES} == PIPELINED


@pytest.mark.parametrize("T,Ci,Co", SHAPES)
def test_poison_build_equals_release(libs, T, Ci, Co):
    sg, L = libs
    note(f"lds poison T={T} Ci={Ci} Co={Co}: {sg.gemm_kernel(T, Ci, Co)}")
    qx, dx, pw = operands(sg, T, Ci, Co, seed=T + Ci)
    ref = sg.gemm(qx, dx, pw)
    ref2 = sg.gemm_unfused(qx, dx, pw)
    got = torch.full_like(ref, float("nan"))
    got2 = torch.full_like(ref, float("nan"))
    run_poison(L, "ptpc_gemm", qx, dx, pw, got)
    ws = torch.empty((T, Co), dtype=torch.float32, device="cuda")
    run_poison(L, "ptpc_gemm_unfused", qx, dx, pw, got2, p(ws))
    torch.cuda.synchronize()
    assert not torch.isnan(got).any() and not torch.isnan(got2).any()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "fused differs"
    assert torch.equal(got2.view(torch.int16), ref2.view(torch.int16)), "two-step differs"


@pytest.mark.parametrize("T,Ci,Co,S", SPLIT_K)
def test_poison_build_split_k(libs, T, Ci, Co, S):
    sg, L = libs
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need > 0 and sg.gemm_ws_splits(T, Ci, Co) == S
    note(f"lds poison split-K T={T} Ci={Ci} Co={Co} S={S}")
    qx, dx, pw = operands(sg, T, Ci, Co, seed=11)
    ref = sg.gemm_ws(qx, dx, pw)
    got = torch.full_like(ref, float("nan"))
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    run_poison(L, "ptpc_gemm_ws", qx, dx, pw, got, p(ws), need)
    torch.cuda.synchronize()
    assert not torch.isnan(got).any()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
