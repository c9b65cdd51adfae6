"""Kernel coverage of the GPU parity cases, checked on the CPU.

The library picks its GEMM and activation-quantization kernels on the host
from the extents alone, and reports the choice through ptpc_gemm_kernel and
ptpc_quant_act_kernel.  Every kernel it can pick must be launched by at
least one GPU parity case (tests/parity_shapes.py), so that no variant
reaches users untested.
"""
import pytest

import parity_shapes

# Every kernel the choice can return (one entry per instantiation).
GEMM_KERNELS = {
    "gemm16_kernel<256,256,2,2>", "gemm16_kernel<192,256,2,2>", "gemm16_kernel<256,224,4,1>",
    "gemm16_kernel<256,160,2,2>", "gemm16_kernel<128,256,2,2>",
    "gemm16_kernel<128,128,2,2>", "gemm16_kernel<128,224,2,2>", "gemm16s_kernel",
    "gemm_kernel<64,64,2,2,4>",
    "gemm_kernel<64,128,2,2,4>", "gemm_kernel<128,128,2,2,4>", "gemm_kernel<32,64,1,2,4>",
    "gemm_decode_kernel<2,2,4,4>", "gemm_decode_kernel<2,1,4,4>",
    "gemm_decode_kernel<1,2,4,4>", "gemm_decode_kernel<1,1,4,4>",
}
ACT_KERNELS = {
    "quant_act_kernel<16,1>", "quant_act_kernel<16,2>", "quant_act_kernel<16,4>",
    "quant_act_kernel<16,8>", "quant_act_kernel<32,8>", "quant_act_kernel<256,1>",
    "quant_act_kernel<256,2>", "quant_act_kernel<128,8>", "quant_act_kernel<256,8>",
    "quant_act_kernel<256,16>", "quant_act_kernel<256,32>", "quant_act_long_kernel",
}


@pytest.fixture(scope="module")
def sg():
    import scaled_gemm_amd
    scaled_gemm_amd.lib()
    return scaled_gemm_amd


def test_choice_is_a_known_kernel(sg):
    """Over a dense grid of shapes the choice only ever names a listed kernel
    (so the lists above are complete)."""
    seen_g, seen_a = set(), set()
    for T in list(range(1, 300)) + [384, 511, 512, 600, 1000, 1024, 2048, 4096, 8192, 16384]:
        for Co in (16, 256, 528, 1040, 4096, 8192, 10240, 14336, 28672, 32768, 57344, 65536):
            for Ci in (16, 4096, 16384):
                seen_g.add(sg.gemm_kernel(T, Ci, Co))
    for Ci in range(16, 70000, 16):
        seen_a.add(sg.quant_act_kernel(4, Ci))
    assert seen_g <= GEMM_KERNELS, seen_g - GEMM_KERNELS
    assert seen_g == GEMM_KERNELS, GEMM_KERNELS - seen_g
    assert seen_a == ACT_KERNELS, seen_a ^ ACT_KERNELS


def test_parity_cases_reach_every_gemm_kernel(sg):
    reached = {sg.gemm_kernel(*s) for s in parity_shapes.gemm_shapes()}
    assert reached == GEMM_KERNELS, f"no parity case launches {sorted(GEMM_KERNELS - reached)}"


def test_parity_cases_reach_every_activation_kernel(sg):
    reached = {sg.quant_act_kernel(*s) for s in parity_shapes.quant_act_shapes()}
    reached.discard("fill_f32_kernel")
    assert reached == ACT_KERNELS, f"no parity case launches {sorted(ACT_KERNELS - reached)}"


def test_queries_reject_what_the_calls_reject(sg):
    assert sg.gemm_kernel(0, 256, 512) is None
    assert sg.gemm_kernel(16, 8, 512) is None          # Ci not a multiple of 16
    assert sg.gemm_kernel(16, (1 << 17) + 16, 512) is None
    assert sg.quant_act_kernel(0, 256) is None
    assert sg.quant_act_kernel(3, 0) == "fill_f32_kernel"


def test_lds_poison_shapes_reach_every_pipelined_kernel(sg):
    """The LDS-poison comparison (a GPU test) runs one shape per pipelined
    kernel; the choice those shapes make is checked here, on the CPU."""
    import test_gpu_lds_poison as poison
    assert {sg.gemm_kernel(*s) for s in poison.SHAPES} == poison.PIPELINED


def test_random_parity_shapes_reach_many_kernels(sg):
    """The seeded random-shape parity test (a GPU test) draws a fixed set of
    shapes; on the CPU: it reaches most GEMM kernel families, and some of
    its shapes make the workspace call split K."""
    import test_gpu_random_shapes as rnd
    assert len({sg.gemm_kernel(*s) for s in rnd.SHAPES}) >= 9
    assert sum(sg.gemm_ws_splits(*s) > 1 for s in rnd.SHAPES) >= 2
