"""The epilogue's fp32 -> bf16 pair conversion on the GPU, exhaustively.

Every fused and two-step epilogue rounds its fp32 results to bf16 through
f32x2_to_bf16x2_rne (device_common.h: gfx950's v_cvt_pk_bf16_f32).  This
runs that device function over all 2^32 fp32 bit patterns in each half of
the pair and compares with integer round-to-nearest-even (NaN in, NaN of the
same sign out); tests/gpu_checks/cvt_bf16_check.hip holds the kernel.
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_bf16_pair_conversion_is_rne_for_every_fp32_pattern():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "gpu_checks"))
    from build_checks import CVT_LIB
    assert os.path.exists(CVT_LIB), "build the test kernels first (__graft_entry__.build)"
    L = ctypes.CDLL(CVT_LIB)
    L.cvt_bf16_check.restype = ctypes.c_int
    L.cvt_bf16_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    res = torch.tensor([0, -1], dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()
    assert L.cvt_bf16_check(ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    bad, first = res.cpu().tolist()
    assert bad == 0, f"{bad} pairs differ from RNE; first low-half pattern {first & 0xFFFFFFFF:#010x}"
