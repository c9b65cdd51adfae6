"""The two-range K join when the other range's flag never comes, through the
C ABI of the lost-flag debug build (libptpc_join_lost.so).

In that build the workgroup that publishes a tile's partial sums never raises
the tile's flag, and the other one waits only 16 sleeps, so every joined tile
takes the path of a wait that runs out.  Its outputs must all be NaN -- never
a sum with whatever partials the workspace still holds from an earlier call
-- and the kernel must exit as usual.  Every path that does not join two
ranges (the plain GEMM, the reduction pass of more ranges) must still equal
the release library bit for bit.
"""
import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

JOINED = (300, 16400, 10768, 2)      # two K ranges of 256x256 tiles, joined in the kernel
REDUCED = (200, 4112, 400, 4)        # four ranges, added by the reduction pass


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_gemm_amd as sg
    from scaled_gemm_amd import build
    sg.lib()
    assert os.path.exists(build.JOIN_LOST_LIB), "build the lost-flag variant first"
    P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L = ctypes.CDLL(build.JOIN_LOST_LIB)
    L.ptpc_gemm.restype = ctypes.c_int
    L.ptpc_gemm.argtypes = [P, I, P, P, P, I, I, I, P, I, P]
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
    x[:, ::43] *= 30
    w = (0.02 * torch.randn((Ci, Co), generator=g, device="cuda")).to(torch.bfloat16)
    qx, dx = sg.quant_act(x)
    return qx, dx, sg.quant_weight(w)


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def call(L, fn, qx, dx, pw, out, *extra):
    T, Ci = qx.shape
    st = getattr(L, fn)(p(qx), Ci, p(dx), p(pw.data), p(pw.dw), T, Ci, pw.Co, p(out), pw.Co,
                        *extra, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"{fn} -> {st}"


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_lost_flag_gives_nan_not_stale_sums(libs):
    sg, L = libs
    T, Ci, Co, S = JOINED
    assert sg.gemm_ws_splits(T, Ci, Co) == S
    note(f"join lost T={T} Ci={Ci} Co={Co} S={S}")
    qx, dx, pw = operands(sg, T, Ci, Co, seed=11)
    ws = torch.empty((sg.gemm_workspace_bytes(T, Ci, Co),), dtype=torch.uint8, device="cuda")
    # the release library leaves this call's published partial sums in the workspace
    ref = sg.gemm_ws(qx, dx, pw, out=torch.empty((T, Co), dtype=torch.bfloat16, device="cuda"),
                     workspace=ws)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    out = torch.zeros((T, Co), dtype=torch.bfloat16, device="cuda")
    call(L, "ptpc_gemm_ws", qx, dx, pw, out, p(ws), ws.numel())
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), f"{int((~torch.isnan(out)).sum())} outputs are not NaN"
    # the same library's plain GEMM is untouched
    plain = torch.full((T, Co), float("nan"), dtype=torch.bfloat16, device="cuda")
    call(L, "ptpc_gemm", qx, dx, pw, plain)
    torch.cuda.synchronize()
    assert same(plain, sg.gemm(qx, dx, pw))


def test_lost_flag_build_keeps_the_reduction_pass(libs):
    sg, L = libs
    T, Ci, Co, S = REDUCED
    assert sg.gemm_ws_splits(T, Ci, Co) == S
    note(f"join lost, reduction pass T={T} Ci={Ci} Co={Co} S={S}")
    qx, dx, pw = operands(sg, T, Ci, Co, seed=12)
    ws = torch.empty((sg.gemm_workspace_bytes(T, Ci, Co),), dtype=torch.uint8, device="cuda")
    ref = sg.gemm_ws(qx, dx, pw, workspace=ws)
    out = torch.full((T, Co), float("nan"), dtype=torch.bfloat16, device="cuda")
    call(L, "ptpc_gemm_ws", qx, dx, pw, out, p(ws), ws.numel())
    torch.cuda.synchronize()
    assert same(out, ref)
