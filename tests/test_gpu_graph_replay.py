"""The split-K GEMM forms under HIP graph capture and replay, through the C ABI.

ptpc_gemm_ws and ptpc_gemm_noalloc keep per-call state on the device: the
reduction-pass form writes every K range's partial sums before adding them,
and the form that joins two K ranges inside the GEMM kernel takes tickets on
per-tile records that a fill kernel clears at the start of each call.  A
graph replays those launches verbatim, so every replay must start from the
same state as an eager call.  Each form is captured once, then replayed
three times with eager calls on other inputs (which leave other values in the
workspace, the records and the outputs) between the replays; every replay
must equal the eager result of the captured inputs bit for bit.
"""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

# (T, Ci, Co, K ranges): the reduction pass over 128x128 tiles, the reduction
# pass over 256x256 tiles, and two ranges joined inside the kernel.
CASES = [(200, 4112, 400, 4), (300, 12304, 528, 8), (300, 16400, 10768, 2)]


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


def operands(sg, T, Ci, Co, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((T, Ci), generator=g, device="cuda").to(torch.bfloat16)
    x[:, ::41] *= 30
    w = (0.02 * torch.randn((Ci, Co), generator=g, device="cuda")).to(torch.bfloat16)
    qx, dx = sg.quant_act(x)
    return qx, dx, sg.quant_weight(w)


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("T,Ci,Co,S", CASES)
@pytest.mark.parametrize("form", ["ws", "noalloc"])
def test_split_k_graph_replays(sg, T, Ci, Co, S, form):
    assert sg.gemm_ws_splits(T, Ci, Co) == S
    note(f"graph replay {form} T={T} Ci={Ci} Co={Co} S={S}")
    qx, dx, pw = operands(sg, T, Ci, Co, seed=T + S)
    qx2, dx2, _ = operands(sg, T, Ci, Co, seed=T + S + 1)
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, Co), dtype=torch.bfloat16, device="cuda")

    def call(a, b):
        if form == "ws":
            sg.gemm_ws(a, b, pw, out=out, workspace=ws)
        else:
            sg.gemm_noalloc(a, b, pw, out=out)

    call(qx2, dx2)
    torch.cuda.synchronize()
    other = out.clone()
    call(qx, dx)
    torch.cuda.synchronize()
    want = out.clone()
    assert not same(want, other)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        call(qx, dx)                    # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            call(qx, dx)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        call(qx2, dx2)                  # eager work between replays: other sums, other records
        torch.cuda.synchronize()
        assert same(out, other), f"eager call before replay {rep}"
        graph.replay()
        torch.cuda.synchronize()
        assert same(out, want), f"replay {rep} differs from the eager result"
    del graph
