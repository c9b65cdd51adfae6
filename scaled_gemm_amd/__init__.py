"""Python binding of libptpc, the PTPC-FP8 hot path for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libptpc.so`` behind the C ABI declared in ``include/ptpc.h``.  PyTorch
provides device memory and the current stream; nothing here computes.  If
the library has not been built, every call raises -- there is no fallback.

Tensors: bf16 inputs as ``torch.bfloat16``; E4M3 codes as ``torch.uint8``
(view as ``torch.float8_e4m3fn`` if wanted); scales ``torch.float32``.
"""
import ctypes
import os
from dataclasses import dataclass

import torch  # must load before libptpc so both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libptpc.so")

_STATUS = {
    0: "PTPC_OK", 1: "PTPC_ERR_NULL", 2: "PTPC_ERR_SHAPE", 3: "PTPC_ERR_UNSUPPORTED",
    4: "PTPC_ERR_ALIGN", 5: "PTPC_ERR_HIP",
}

# Every symbol include/ptpc.h declares.
EXPORTS = (
    "ptpc_status_string", "ptpc_abi_version", "ptpc_quant_act", "ptpc_weight_packed_bytes",
    "ptpc_quant_weight", "ptpc_unpack_weight", "ptpc_gemm",
    "ptpc_gemm_workspace_bytes", "ptpc_gemm_ws", "ptpc_gemm_noalloc",
    "ptpc_gemm_unfused_workspace_bytes", "ptpc_gemm_unfused",
    "ptpc_gemm_unfused_bf16_workspace_bytes", "ptpc_gemm_unfused_bf16", "ptpc_tensor_scale",
    "ptpc_quant_act_static", "ptpc_quant_weight_static", "ptpc_gemm_tensor",
    "ptpc_gemm_kernel", "ptpc_quant_act_kernel", "ptpc_gemm_ws_splits",
)

_lib = None


class PtpcError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def lib():
    """The loaded libptpc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_gemm_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.ptpc_status_string.restype = ctypes.c_char_p
        L.ptpc_status_string.argtypes = [ctypes.c_int]
        L.ptpc_abi_version.restype = ctypes.c_int
        L.ptpc_abi_version.argtypes = []
        L.ptpc_quant_act.restype = ctypes.c_int
        L.ptpc_quant_act.argtypes = [P, I, I, I, P, I, P, P]
        L.ptpc_weight_packed_bytes.restype = S
        L.ptpc_weight_packed_bytes.argtypes = [I, I]
        L.ptpc_quant_weight.restype = ctypes.c_int
        L.ptpc_quant_weight.argtypes = [P, I, I, I, P, P, P]
        L.ptpc_unpack_weight.restype = ctypes.c_int
        L.ptpc_unpack_weight.argtypes = [P, I, I, P, P]
        L.ptpc_gemm.restype = ctypes.c_int
        L.ptpc_gemm.argtypes = [P, I, P, P, P, I, I, I, P, I, P]
        L.ptpc_gemm_unfused_workspace_bytes.restype = S
        L.ptpc_gemm_unfused_workspace_bytes.argtypes = [I, I]
        L.ptpc_gemm_unfused.restype = ctypes.c_int
        L.ptpc_gemm_unfused.argtypes = [P, I, P, P, P, I, I, I, P, I, P, P]
        L.ptpc_gemm_workspace_bytes.restype = S
        L.ptpc_gemm_workspace_bytes.argtypes = [I, I, I]
        L.ptpc_gemm_ws.restype = ctypes.c_int
        L.ptpc_gemm_ws.argtypes = [P, I, P, P, P, I, I, I, P, I, P, S, P]
        L.ptpc_gemm_noalloc.restype = ctypes.c_int
        L.ptpc_gemm_noalloc.argtypes = [P, I, P, P, P, I, I, I, P, I, P]
        L.ptpc_gemm_unfused_bf16_workspace_bytes.restype = S
        L.ptpc_gemm_unfused_bf16_workspace_bytes.argtypes = [I, I]
        L.ptpc_gemm_unfused_bf16.restype = ctypes.c_int
        L.ptpc_gemm_unfused_bf16.argtypes = [P, I, P, P, P, I, I, I, P, I, P, P]
        L.ptpc_tensor_scale.restype = ctypes.c_int
        L.ptpc_tensor_scale.argtypes = [P, I, I, I, P, P]
        L.ptpc_quant_act_static.restype = ctypes.c_int
        L.ptpc_quant_act_static.argtypes = [P, I, I, I, P, P, I, P]
        L.ptpc_quant_weight_static.restype = ctypes.c_int
        L.ptpc_quant_weight_static.argtypes = [P, I, I, I, P, P, P]
        L.ptpc_gemm_tensor.restype = ctypes.c_int
        L.ptpc_gemm_tensor.argtypes = [P, I, P, P, P, I, I, I, P, I, P]
        L.ptpc_gemm_kernel.restype = ctypes.c_char_p
        L.ptpc_gemm_kernel.argtypes = [I, I, I]
        L.ptpc_quant_act_kernel.restype = ctypes.c_char_p
        L.ptpc_quant_act_kernel.argtypes = [I, I]
        L.ptpc_gemm_ws_splits.restype = ctypes.c_int
        L.ptpc_gemm_ws_splits.argtypes = [I, I, I]
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise PtpcError(fn, status)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


# Every tensor handed to the library is checked here before the call: the
# kernels trust the extents they are given, so a buffer that is too small or
# not on the GPU would be read or written out of bounds on the device.
def _on_gpu(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a tensor on the GPU, got one on {t.device}")


def _matrix(t, dtype, name, shape=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a 2-D tensor with unit column stride")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    _on_gpu(t, name)
    return t.shape[0], t.shape[1], max(t.stride(0), t.shape[1])


def _vector(t, n, dtype, name, exact=True):
    """A contiguous 1-D buffer of n (exact) or at least n elements."""
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 1-D tensor")
    if (t.numel() != n) if exact else (t.numel() < n):
        want = f"{n}" if exact else f"at least {n}"
        raise ValueError(f"{name}: expected {want} elements, got {t.numel()}")
    _on_gpu(t, name)


def _scratch(t, nbytes, name):
    """A contiguous buffer of at least nbytes bytes, any dtype."""
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: expected at least {nbytes} bytes, got "
                         f"{t.numel() * t.element_size()}")
    _on_gpu(t, name)


def packed_bytes(Ci: int, Co: int) -> int:
    return int(lib().ptpc_weight_packed_bytes(Ci, Co))


def workspace_bytes(T: int, Co: int) -> int:
    return int(lib().ptpc_gemm_unfused_workspace_bytes(T, Co))


@dataclass
class PackedWeight:
    """A weight quantized once: packed E4M3 codes plus its scales -- one per
    output column (per-channel, from quant_weight) or, with per_tensor set,
    one for the whole matrix (from quant_weight_static)."""
    data: torch.Tensor     # uint8 [packed_bytes(Ci, Co)]
    dw: torch.Tensor       # float32 [Co], or [1] when per_tensor
    Ci: int
    Co: int
    per_tensor: bool = False


def _check_packed(pw: PackedWeight, name, per_tensor):
    if pw.per_tensor != per_tensor:
        kind = "per-tensor" if pw.per_tensor else "per-channel"
        raise ValueError(f"{name}: got a {kind} weight; this call needs "
                         f"{'a per-tensor' if per_tensor else 'a per-channel'} one")
    _vector(pw.data, packed_bytes(pw.Ci, pw.Co), torch.uint8, f"{name}.data", exact=False)
    _vector(pw.dw, 1 if per_tensor else pw.Co, torch.float32, f"{name}.dw")


def gemm_kernel(T: int, Ci: int, Co: int):
    """Name of the GEMM kernel ptpc_gemm launches for this shape (None if none)."""
    r = lib().ptpc_gemm_kernel(T, Ci, Co)
    return r.decode() if r is not None else None


def gemm_ws_splits(T: int, Ci: int, Co: int) -> int:
    """K ranges ptpc_gemm_ws / ptpc_gemm_noalloc use for this shape (1: no split)."""
    return int(lib().ptpc_gemm_ws_splits(T, Ci, Co))


def quant_act_kernel(T: int, Ci: int):
    """Name of the kernel ptpc_quant_act launches for T rows of Ci elements."""
    r = lib().ptpc_quant_act_kernel(T, Ci)
    return r.decode() if r is not None else None


def quant_act(x, qx=None, dx=None, stream=None):
    """Per-token FP8 quantization of bf16 X [T, Ci] -> (codes uint8 [T, Ci], dx fp32 [T])."""
    T, Ci, ldx = _matrix(x, torch.bfloat16, "x")
    if qx is None:
        qx = torch.empty((T, Ci), dtype=torch.uint8, device=x.device)
    if dx is None:
        dx = torch.empty((T,), dtype=torch.float32, device=x.device)
    _, _, ldq = _matrix(qx, torch.uint8, "qx", (T, Ci))
    _vector(dx, T, torch.float32, "dx")
    _check("ptpc_quant_act", lib().ptpc_quant_act(_ptr(x), T, Ci, ldx, _ptr(qx), ldq, _ptr(dx),
                                                  _stream(stream)))
    return qx, dx


def quant_weight(w, out: PackedWeight = None, stream=None) -> PackedWeight:
    """Per-output-channel FP8 quantization + MFMA prepack of bf16 W [Ci, Co]."""
    Ci, Co, ldw = _matrix(w, torch.bfloat16, "w")
    if out is None:
        out = PackedWeight(torch.empty((packed_bytes(Ci, Co),), dtype=torch.uint8, device=w.device),
                           torch.empty((Co,), dtype=torch.float32, device=w.device), Ci, Co)
    if (out.Ci, out.Co) != (Ci, Co):
        raise ValueError(f"out: PackedWeight is {out.Ci}x{out.Co}, w is {Ci}x{Co}")
    _check_packed(out, "out", per_tensor=False)
    _check("ptpc_quant_weight", lib().ptpc_quant_weight(_ptr(w), Ci, Co, ldw, _ptr(out.data),
                                                        _ptr(out.dw), _stream(stream)))
    return out


def unpack_weight(pw: PackedWeight, stream=None):
    """E4M3 codes of the weight back in [Ci, Co] order (for tests)."""
    _vector(pw.data, packed_bytes(pw.Ci, pw.Co), torch.uint8, "pw.data", exact=False)
    qw = torch.empty((pw.Ci, pw.Co), dtype=torch.uint8, device=pw.data.device)
    _check("ptpc_unpack_weight", lib().ptpc_unpack_weight(_ptr(pw.data), pw.Ci, pw.Co, _ptr(qw),
                                                          _stream(stream)))
    return qw


def _gemm_args(qx, dx, pw: PackedWeight, out, per_tensor):
    T, Ci, ldq = _matrix(qx, torch.uint8, "qx")
    if Ci != pw.Ci:
        raise ValueError(f"qx has Ci={Ci}, weight has Ci={pw.Ci}")
    _check_packed(pw, "pw", per_tensor)
    if per_tensor:
        _vector(dx, 1, torch.float32, "dx")
    else:
        _vector(dx, T, torch.float32, "dx")
    if out is None:
        out = torch.empty((T, pw.Co), dtype=torch.bfloat16, device=qx.device)
    _matrix(out, torch.bfloat16, "out", (T, pw.Co))
    return T, Ci, ldq, out


def gemm(qx, dx, pw: PackedWeight, out=None, stream=None):
    """Fused PTPC GEMM: bf16 [T, Co] = ((qx @ qw) * dx[:, None]) * dw[None, :]."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=False)
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm", lib().ptpc_gemm(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data), _ptr(pw.dw), T,
                                        Ci, pw.Co, _ptr(out), ldo, _stream(stream)))
    return out


def gemm_workspace_bytes(T: int, Ci: int, Co: int) -> int:
    return int(lib().ptpc_gemm_workspace_bytes(T, Ci, Co))


def gemm_ws(qx, dx, pw: PackedWeight, out=None, workspace=None, stream=None):
    """ptpc_gemm_ws: the fused GEMM, splitting K across workgroups where the
    output tiles alone leave the GPU idle (workspace: uint8 tensor of at least
    gemm_workspace_bytes(T, Ci, Co) bytes; allocated here if not given)."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=False)
    need = gemm_workspace_bytes(T, Ci, pw.Co)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=qx.device)
    if workspace is not None:
        _scratch(workspace, need, "workspace")
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm_ws", lib().ptpc_gemm_ws(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data), _ptr(pw.dw),
                                              T, Ci, pw.Co, _ptr(out), ldo, _ptr(workspace),
                                              nbytes, _stream(stream)))
    return out


# Scratch bytes the library holds per GPU for gemm_noalloc (include/ptpc.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def gemm_noalloc(qx, dx, pw: PackedWeight, out=None, stream=None):
    """ptpc_gemm_noalloc: gemm_ws without a workspace -- the split-K partials
    go to the library's own per-GPU scratch, nothing is allocated (pass `out`
    to allocate nothing here either).  Calls overlapping on one GPU race."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=False)
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm_noalloc",
           lib().ptpc_gemm_noalloc(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data), _ptr(pw.dw), T, Ci,
                                   pw.Co, _ptr(out), ldo, _stream(stream)))
    return out


def gemm_unfused(qx, dx, pw: PackedWeight, out=None, workspace=None, stream=None):
    """Two-step form: fp32 GEMM result to `workspace`, then a rescale pass."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=False)
    if workspace is None:
        workspace = torch.empty((T, pw.Co), dtype=torch.float32, device=qx.device)
    if workspace.dtype != torch.float32:
        raise TypeError(f"workspace: expected torch.float32, got {workspace.dtype}")
    _scratch(workspace, workspace_bytes(T, pw.Co), "workspace")
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm_unfused",
           lib().ptpc_gemm_unfused(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data), _ptr(pw.dw), T, Ci,
                                   pw.Co, _ptr(out), ldo, _ptr(workspace), _stream(stream)))
    return out


def gemm_unfused_bf16(qx, dx, pw: PackedWeight, out=None, workspace=None, stream=None):
    """Two-step form with a bf16 intermediate: bf16(acc) to `workspace`, then scaled."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=False)
    if workspace is None:
        workspace = torch.empty((T, pw.Co), dtype=torch.bfloat16, device=qx.device)
    if workspace.dtype != torch.bfloat16:
        raise TypeError(f"workspace: expected torch.bfloat16, got {workspace.dtype}")
    _scratch(workspace, 2 * T * pw.Co, "workspace")
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm_unfused_bf16",
           lib().ptpc_gemm_unfused_bf16(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data), _ptr(pw.dw), T,
                                        Ci, pw.Co, _ptr(out), ldo, _ptr(workspace),
                                        _stream(stream)))
    return out


def linear(x, pw: PackedWeight, stream=None):
    """Per-token quantization of X followed by the fused GEMM (one layer's forward)."""
    qx, dx = quant_act(x, stream=stream)
    return gemm(qx, dx, pw, stream=stream)


# -- per-tensor comparator ------------------------------------------------------
def tensor_scale(x, d=None, stream=None):
    """One scale for a whole bf16 matrix: d[0] = max|x| / 448 (1 if zero) -> fp32 [1]."""
    R, C, ld = _matrix(x, torch.bfloat16, "x")
    if d is None:
        d = torch.empty((1,), dtype=torch.float32, device=x.device)
    _vector(d, 1, torch.float32, "d")
    _check("ptpc_tensor_scale", lib().ptpc_tensor_scale(_ptr(x), R, C, ld, _ptr(d),
                                                        _stream(stream)))
    return d


def quant_act_static(x, d, qx=None, stream=None):
    """Per-tensor FP8 codes of bf16 X [T, Ci] with the given scale d (fp32 [1])."""
    T, Ci, ldx = _matrix(x, torch.bfloat16, "x")
    if qx is None:
        qx = torch.empty((T, Ci), dtype=torch.uint8, device=x.device)
    _, _, ldq = _matrix(qx, torch.uint8, "qx", (T, Ci))
    _vector(d, 1, torch.float32, "d")
    _check("ptpc_quant_act_static",
           lib().ptpc_quant_act_static(_ptr(x), T, Ci, ldx, _ptr(d), _ptr(qx), ldq,
                                       _stream(stream)))
    return qx


def quant_weight_static(w, d, out: PackedWeight = None, stream=None) -> PackedWeight:
    """Per-tensor FP8 codes of bf16 W [Ci, Co] with the scale d (fp32 [1]), prepacked;
    the returned PackedWeight carries d as its (one-element) dw and is marked
    per_tensor (only gemm_tensor accepts it)."""
    Ci, Co, ldw = _matrix(w, torch.bfloat16, "w")
    _vector(d, 1, torch.float32, "d")
    if out is None:
        out = PackedWeight(torch.empty((packed_bytes(Ci, Co),), dtype=torch.uint8, device=w.device),
                           d, Ci, Co, per_tensor=True)
    if (out.Ci, out.Co) != (Ci, Co):
        raise ValueError(f"out: PackedWeight is {out.Ci}x{out.Co}, w is {Ci}x{Co}")
    _check_packed(out, "out", per_tensor=True)
    _check("ptpc_quant_weight_static",
           lib().ptpc_quant_weight_static(_ptr(w), Ci, Co, ldw, _ptr(d), _ptr(out.data),
                                          _stream(stream)))
    return out


def gemm_tensor(qx, dx, pw: PackedWeight, out=None, stream=None):
    """Per-tensor FP8 GEMM: bf16 [T, Co] = ((qx @ qw) * dx[0]) * dw[0]."""
    T, Ci, ldq, out = _gemm_args(qx, dx, pw, out, per_tensor=True)
    ldo = max(out.stride(0), out.shape[1])
    _check("ptpc_gemm_tensor", lib().ptpc_gemm_tensor(_ptr(qx), ldq, _ptr(dx), _ptr(pw.data),
                                                      _ptr(pw.dw), T, Ci, pw.Co, _ptr(out), ldo,
                                                      _stream(stream)))
    return out
