"""The C ABI of libptpc on the CPU: the library loads, exports every symbol
include/ptpc.h declares, and rejects bad arguments before touching the GPU
(no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ptpc.h")


@pytest.fixture(scope="module")
def L():
    import scaled_gemm_amd as sg
    return sg.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ptpc_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    import scaled_gemm_amd as sg
    assert declared_functions() == sorted(sg.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    import scaled_gemm_amd as sg
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert L.ptpc_abi_version() == 1
    for s in range(6):
        assert L.ptpc_status_string(s).startswith(b"PTPC_")
    assert L.ptpc_status_string(99) == b"unknown ptpc_status"


def test_size_queries(L):
    assert L.ptpc_weight_packed_bytes(256, 512) == 512 * 256
    assert L.ptpc_weight_packed_bytes(1040, 32) == 32 * 1152
    assert L.ptpc_weight_packed_bytes(8, 16) == 0          # Ci not a multiple of 16
    assert L.ptpc_weight_packed_bytes(0, 16) == 0
    assert L.ptpc_gemm_unfused_workspace_bytes(3, 16) == 3 * 16 * 4
    assert L.ptpc_gemm_unfused_workspace_bytes(0, 16) == 0


# Aligned, non-NULL fake device addresses.  Validation must reject before any
# HIP call, and the fault-injection path returns before any launch, so these
# are never dereferenced.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
D = ctypes.c_void_p(0x40000)
E = ctypes.c_void_p(0x50000)
MIS = ctypes.c_void_p(0x10008)
NULL = None


def test_quant_act_validation(L):
    f = L.ptpc_quant_act
    assert f(A, 0, 256, 256, B, 256, C, None) == 0                 # empty: no-op
    assert f(A, -1, 256, 256, B, 256, C, None) == 2
    assert f(A, 4, 256, 128, B, 256, C, None) == 2                 # ldx < Ci
    assert f(A, 4, 256, 256, B, 128, C, None) == 2                 # ldq < Ci
    assert f(A, 4, 24, 24, B, 32, C, None) == 3                    # Ci % 16
    assert f(NULL, 4, 256, 256, B, 256, C, None) == 1
    assert f(A, 4, 256, 256, NULL, 256, C, None) == 1
    assert f(A, 4, 256, 256, B, 256, NULL, None) == 1
    assert f(MIS, 4, 256, 256, B, 256, C, None) == 4
    assert f(A, 4, 256, 260, B, 256, C, None) == 4                 # pitch not 16 B
    assert f(A, 4, 256, 256, B, 264, C, None) == 4


def test_quant_weight_validation(L):
    f = L.ptpc_quant_weight
    assert f(A, 256, 0, 0, B, C, None) == 0
    assert f(A, 256, 512, 500, B, C, None) == 2
    assert f(A, 250, 512, 512, B, C, None) == 3
    assert f(A, 256, 520, 520, B, C, None) == 3
    assert f(NULL, 256, 512, 512, B, C, None) == 1
    assert f(A, 256, 512, 512, NULL, C, None) == 1
    assert f(A, 256, 512, 512, B, NULL, None) == 1
    assert f(A, 256, 512, 512, MIS, C, None) == 4
    assert L.ptpc_unpack_weight(NULL, 256, 512, B, None) == 1
    assert L.ptpc_unpack_weight(A, 256, 500, B, None) == 3
    # K beyond 2^17 (the GEMM's limit) is refused before anything is
    # launched, by every weight call and the size query
    big = (1 << 17) + 16
    assert f(A, big, 512, 512, B, C, None) == 3
    assert L.ptpc_quant_weight_static(A, big, 512, 512, B, C, None) == 3
    assert L.ptpc_unpack_weight(A, big, 512, B, None) == 3
    assert L.ptpc_weight_packed_bytes(big, 512) == 0
    assert L.ptpc_weight_packed_bytes(1 << 17, 512) == 512 << 17


def test_gemm_validation(L):
    for unfused in (False, True):
        def f(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, ws=D):
            if unfused:
                return L.ptpc_gemm_unfused(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, ws, None)
            return L.ptpc_gemm(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, None)
        assert f(A, 256, B, C, D, 0, 256, 512, E, 512) == 0
        assert f(A, 256, B, C, D, 4, 256, 512, E, 500) == 2
        assert f(A, 100, B, C, D, 4, 256, 512, E, 512) == 2
        assert f(A, 256, B, C, D, 4, 256, 500, E, 512) == 3
        assert f(NULL, 256, B, C, D, 4, 256, 512, E, 512) == 1
        assert f(A, 256, NULL, C, D, 4, 256, 512, E, 512) == 1
        assert f(A, 256, B, NULL, D, 4, 256, 512, E, 512) == 1
        assert f(A, 256, B, C, NULL, 4, 256, 512, E, 512) == 1
        assert f(A, 256, B, C, D, 4, 256, 512, NULL, 512) == 1
        assert f(MIS, 256, B, C, D, 4, 256, 512, E, 512) == 4
        assert f(A, 256, B, C, D, 4, 256, 512, E, 516) == 4
        assert f(A, (1 << 22) + 16, B, C, D, 4, 256, 512, E, 512) == 3      # ldq > 2^22
        assert f(A, (1 << 17) + 16, B, C, D, 4, (1 << 17) + 16, 512, E, 512) == 3   # Ci > 2^17
        assert f(A, 256, B, C, D, 4, 256, 512, E, (1 << 22) + 16) == 3      # ldo > 2^22
    assert L.ptpc_gemm_unfused(A, 256, B, C, D, 4, 256, 512, E, 512, NULL, None) == 1
    assert L.ptpc_gemm_unfused_bf16(A, 256, B, C, D, 4, 256, 512, E, 512, NULL, None) == 1
    assert L.ptpc_gemm_unfused_bf16(A, 256, B, C, D, 4, 256, 512, E, 512, MIS, None) == 4
    assert L.ptpc_gemm_unfused_bf16(A, 256, B, C, D, 4, 256, 500, E, 512, D, None) == 3
    assert L.ptpc_gemm_unfused_bf16_workspace_bytes(3, 16) == 3 * 16 * 2
    # split-K workspace: 128 tokens x 8192 -> 10240 columns splits K three ways
    need = L.ptpc_gemm_workspace_bytes(128, 8192, 10240)
    assert need == 3 * 4 * 128 * 10240
    assert L.ptpc_gemm_workspace_bytes(4096, 28672, 8192) == 0          # enough tiles
    assert L.ptpc_gemm_workspace_bytes(16, 8192, 8192) == 0             # few-token kernel
    assert L.ptpc_gemm_workspace_bytes(128, 8192, 57344) == 0           # 448 tiles
    assert L.ptpc_gemm_workspace_bytes(128, 8192, 8192) == 0            # K split in-workgroup
    assert L.ptpc_gemm_workspace_bytes(128, 28672, 8192) == 4 * 4 * 128 * 8192  # long K: split
    # from 256 tokens: 256x256 tiles, S = 256 // tiles (<= 8), K >= 12288 only
    assert L.ptpc_gemm_workspace_bytes(256, 28672, 8192) == 8 * 4 * 256 * 8192   # 32 tiles
    # two ranges over 256x256 tiles are joined in the GEMM kernel: one fp32
    # slot of 256x256 per tile and a 16-byte record per tile
    assert L.ptpc_gemm_workspace_bytes(1024, 28672, 8192) == 128 * (4 * 256 * 256 + 16)
    assert L.ptpc_gemm_workspace_bytes(1024, 14336, 4096) == 4 * 4 * 1024 * 4096  # 64 tiles
    assert L.ptpc_gemm_workspace_bytes(256, 14336, 4096) == 8 * 4 * 256 * 4096    # 16 tiles
    assert L.ptpc_gemm_workspace_bytes(512, 14336, 4096) == 0    # K < 16384, 64x128 fill the GPU
    assert L.ptpc_gemm_workspace_bytes(2048, 14336, 4096) == 0   # K < 16384, 2 ranges only
    assert L.ptpc_gemm_workspace_bytes(2048, 28672, 4096) == 128 * (4 * 256 * 256 + 16)  # long K: 2
    assert L.ptpc_gemm_workspace_bytes(300, 16400, 10768) == 86 * (4 * 256 * 256 + 16)  # ragged: 2
    # the split count behind those sizes (1: no split; 0: rejected shape)
    sp = L.ptpc_gemm_ws_splits
    assert [sp(1024, 28672, 8192), sp(256, 28672, 8192), sp(128, 8192, 10240),
            sp(4096, 28672, 8192), sp(300, 16400, 10768)] == [2, 8, 3, 1, 2]
    assert sp(0, 256, 256) == 0 and sp(16, 250, 256) == 0 and sp(16, 256, 0) == 0
    # 129..255 tokens: one 256-row tile (the weight read once) for long K or
    # where ptpc_gemm would run 128x128 tiles, else 128x128 split tiles
    assert L.ptpc_gemm_workspace_bytes(200, 28672, 8192) == 8 * 4 * 200 * 8192   # long K
    assert L.ptpc_gemm_workspace_bytes(200, 8192, 10240) == 6 * 4 * 200 * 10240  # 128x128 plan
    assert L.ptpc_gemm_workspace_bytes(200, 8192, 8192) == 2 * 4 * 200 * 8192    # 128x128 split
    assert L.ptpc_gemm_workspace_bytes(1024, 8192, 8192) == 0            # short K
    assert L.ptpc_gemm_workspace_bytes(2048, 28672, 8192) == 0           # 256 tiles
    assert L.ptpc_gemm_workspace_bytes(300, 1024, 256) == 0              # short K
    assert L.ptpc_gemm_workspace_bytes(300, 2048 * 6, 256) == 8 * 4 * 300 * 256   # >= 8 steps each
    g = L.ptpc_gemm_ws
    assert g(A, 8192, B, C, D, 128, 8192, 10240, E, 10240, NULL, 0, None) == 1
    assert g(A, 8192, B, C, D, 128, 8192, 10240, E, 10240, D, need - 16, None) == 2
    assert g(A, 8192, B, C, D, 128, 8192, 10240, E, 10240, MIS, need, None) == 4
    assert g(A, 256, B, C, D, 4, 256, 500, E, 512, D, 0, None) == 3
    assert L.ptpc_gemm_unfused(A, 256, B, C, D, 4, 256, 512, E, 512, MIS, None) == 4


def test_per_tensor_validation(L):
    ts, qa, qw, gt = (L.ptpc_tensor_scale, L.ptpc_quant_act_static, L.ptpc_quant_weight_static,
                      L.ptpc_gemm_tensor)
    assert ts(A, 4, 256, 128, B, None) == 2                        # ld < C
    assert ts(A, -1, 256, 256, B, None) == 2
    assert ts(A, 4, 24, 24, B, None) == 3
    assert ts(A, 4, 256, 256, NULL, None) == 1
    assert ts(NULL, 4, 256, 256, B, None) == 1
    assert ts(MIS, 4, 256, 256, B, None) == 4
    assert ts(A, 4, 256, 260, B, None) == 4
    assert qa(A, 0, 256, 256, B, C, 256, None) == 0                # empty: no-op
    assert qa(A, 4, 256, 256, NULL, C, 256, None) == 1             # scale pointer
    assert qa(A, 4, 256, 256, B, NULL, 256, None) == 1
    assert qa(A, 4, 256, 256, B, C, 128, None) == 2
    assert qa(A, 4, 24, 24, B, C, 32, None) == 3
    assert qa(A, 4, 256, 256, MIS, C, 256, None) == 4
    assert qw(A, 256, 0, 0, B, C, None) == 0
    assert qw(A, 256, 512, 500, B, C, None) == 2
    assert qw(A, 256, 520, 520, B, C, None) == 3
    assert qw(A, 256, 512, 512, NULL, C, None) == 1
    assert qw(A, 256, 512, 512, B, MIS, None) == 4
    assert gt(A, 256, B, C, D, 0, 256, 512, E, 512, None) == 0
    assert gt(A, 256, B, C, D, 4, 256, 500, E, 512, None) == 3
    assert gt(A, 256, NULL, C, D, 4, 256, 512, E, 512, None) == 1
    assert gt(A, 256, B, C, NULL, 4, 256, 512, E, 512, None) == 1
    assert gt(A, 256, B, C, D, 4, 256, 512, E, 516, None) == 4


def test_forced_launch_failure_reports_hip_error():
    """PTPC_FAULT=launch makes every launching call return PTPC_ERR_HIP from
    the host, without a GPU; checked in a child process so the setting does
    not leak into other tests."""
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import scaled_gemm_amd as sg
L = sg.lib()
A, B, C, D, E = (ctypes.c_void_p(v) for v in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
r = [L.ptpc_quant_act(A, 4, 256, 256, B, 256, C, None),
     L.ptpc_quant_weight(A, 256, 512, 512, B, C, None),
     L.ptpc_unpack_weight(A, 256, 512, B, None),
     L.ptpc_gemm(A, 256, B, C, D, 4, 256, 512, E, 512, None),
     L.ptpc_gemm_unfused(A, 256, B, C, D, 4, 256, 512, E, 512, D, None),
     L.ptpc_tensor_scale(A, 4, 256, 256, B, None),
     L.ptpc_quant_act_static(A, 4, 256, 256, B, C, 256, None),
     L.ptpc_quant_weight_static(A, 256, 512, 512, B, C, None),
     L.ptpc_gemm_tensor(A, 256, B, C, D, 4, 256, 512, E, 512, None),
     L.ptpc_gemm_unfused_bf16(A, 256, B, C, D, 4, 256, 512, E, 512, D, None),
     L.ptpc_gemm_ws(A, 8192, B, C, D, 128, 8192, 10240, E, 10240, D, 1 << 30, None),
     L.ptpc_gemm_noalloc(A, 8192, B, C, D, 128, 8192, 10240, E, 10240, None),
     L.ptpc_quant_act(A, 0, 256, 256, B, 256, C, None)]
print(r)
assert r == [5, 5, 5, 5, 5, 5, 5, 5, 5, 5, 5, 5, 0], r
""" % ROOT
    env = dict(os.environ, PTPC_FAULT="launch", HIP_VISIBLE_DEVICES="")
    subprocess.run(["python", "-c", code], check=True, env=env)


def test_noalloc_scratch_covers_every_split(L):
    """ptpc_gemm_noalloc's per-GPU scratch holds the partial sums of every
    shape the split-K plan splits (64 MiB by construction: 128x128 splits
    need at most 16 MiB, 256x256 splits at most 64 MiB), and the call
    validates like ptpc_gemm (no compute call here)."""
    import scaled_gemm_amd as sg
    assert sg.NOALLOC_SCRATCH_BYTES == 64 << 20
    worst = max(L.ptpc_gemm_workspace_bytes(T, Ci, Co) for T in range(65, 129)
                for Ci in (2048, 8192, 28672) for Co in range(16, 66000, 16))
    assert 0 < worst <= 16 << 20
    worst = max(L.ptpc_gemm_workspace_bytes(T, Ci, Co) for T in range(129, 256)
                for Ci in (2048, 8192, 28672) for Co in range(16, 66000, 16))
    assert 16 << 20 < worst <= sg.NOALLOC_SCRATCH_BYTES
    worst = max(L.ptpc_gemm_workspace_bytes(T, Ci, Co)
                for T in list(range(256, 1100, 7)) + [1536, 2048, 4096, 8192, 16384]
                for Ci in (8192, 12288, 14336, 28672, 65536) for Co in range(16, 66000, 48))
    assert 16 << 20 < worst <= sg.NOALLOC_SCRATCH_BYTES
    f = L.ptpc_gemm_noalloc
    assert f(A, 256, B, C, D, 0, 256, 512, E, 512, None) == 0
    assert f(A, 256, B, C, D, 4, 256, 500, E, 512, None) == 3
    assert f(NULL, 256, B, C, D, 4, 256, 512, E, 512, None) == 1
    assert f(A, 256, B, C, D, 4, 256, 512, E, 516, None) == 4


def test_debug_builds_export_the_abi():
    """The two debug builds export every symbol of include/ptpc.h, and the
    timeline build also the call of include/ptpc_debug.h."""
    from scaled_gemm_amd import build
    dbg = sorted(set(re.findall(r"\b(ptpc_[a-z0-9_]+)\s*\(",
                                open(os.path.join(ROOT, "include", "ptpc_debug.h")).read())))
    assert dbg == ["ptpc_debug_set_timeline"]
    for lib, extra in ((build.POISON_LIB, []), (build.TIMELINE_LIB, dbg)):
        out = subprocess.run(["nm", "-D", "--defined-only", lib], check=True,
                             stdout=subprocess.PIPE, text=True).stdout
        exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
        for name in declared_functions() + extra:
            assert name in exported, (lib, name)
