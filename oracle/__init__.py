"""CPU oracle for the PTPC-FP8 hot path -- TEST INFRASTRUCTURE ONLY.

The plain, slow definition of what the GPU library computes, checked against
the pins in ``tests/test_oracle_*.py``.  Only the tests, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package; the
product package never does, and the two share no code.

Source: vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm"
(2025-02-24).  Arrays: bf16 values are ``numpy.uint16`` bit patterns, E4M3
codes ``numpy.uint8`` bit patterns, scales ``numpy.float32``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load (building first if needed) the compiled oracle."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = ctypes.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int64


def _declare(L):
    L.orc_e4m3_decode.restype = ctypes.c_double
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_encode_array.argtypes = [_P, _I, _P]
    L.orc_bf16_from_double_array.argtypes = [_P, _I, _P]
    L.orc_quant_act.argtypes = [_P, _I, _I, _I, _P, _I, _P]
    L.orc_quant_weight.argtypes = [_P, _I, _I, _I, _P, _I, _P]
    L.orc_quant_tensor.argtypes = [_P, _I, _I, _I, _P, _I, _P]
    L.orc_quant_static.argtypes = [_P, _I, _I, _I, ctypes.c_float, _P, _I]
    L.orc_gemm_exact.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P]
    L.orc_gemm_exact_i64.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P]
    L.orc_gemm_exact_sampled.argtypes = [_P, _I, _P, _I, _I, _P, _P, _I, _P]
    L.orc_apply_scales.argtypes = [_P, _I, _I, _P, _P, _P]
    L.orc_apply_scales_sampled.argtypes = [_P, _P, _P, _I, _P, _P, _P]
    L.orc_gemm_dequant_first.argtypes = [_P, _I, _P, _P, _I, _P, _I, _I, _I, _P]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_num_threads.argtypes = []


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def num_threads() -> int:
    return lib().orc_num_threads()


# -- E4M3 codec -------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """Value (float64) of each E4M3 code; NaN for 0x7F / 0xFF."""
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    table = np.array([L.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e4m3_encode(f) -> np.ndarray:
    """Round-to-nearest-even, saturating E4M3 code of each fp32 value."""
    f = _c(np.asarray(f, dtype=np.float32), np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(f), f.size, _ptr(out))
    return out


def bf16_from_double(v) -> np.ndarray:
    """Nearest bf16 (ties to even) of each double, as uint16 bits."""
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_from_double_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# -- quantizers ---------------------------------------------------------------
def quant_act(x):
    """Per-token quantization of X [T, Ci] (bf16 bits) -> (codes [T, Ci], dx [T])."""
    x = _c(x, np.uint16)
    T, Ci = x.shape
    q = np.empty((T, Ci), dtype=np.uint8)
    d = np.empty(T, dtype=np.float32)
    lib().orc_quant_act(_ptr(x), T, Ci, Ci, _ptr(q), Ci, _ptr(d))
    return q, d


def quant_weight(w):
    """Per-output-channel quantization of W [Ci, Co] -> (codes [Ci, Co], dw [Co])."""
    w = _c(w, np.uint16)
    Ci, Co = w.shape
    q = np.empty((Ci, Co), dtype=np.uint8)
    d = np.empty(Co, dtype=np.float32)
    lib().orc_quant_weight(_ptr(w), Ci, Co, Co, _ptr(q), Co, _ptr(d))
    return q, d


def quant_tensor(x):
    """Per-tensor quantization (one scale for the whole tensor)."""
    x = _c(x, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), dtype=np.uint8)
    d = np.empty(1, dtype=np.float32)
    lib().orc_quant_tensor(_ptr(x), R, C, C, _ptr(q), C, _ptr(d))
    return q, d[0]


def quant_static(x, s):
    """Static per-tensor quantization with the given scalar scale s."""
    x = _c(x, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), dtype=np.uint8)
    lib().orc_quant_static(_ptr(x), R, C, C, ctypes.c_float(float(s)), _ptr(q), C)
    return q


# -- contraction and scales ------------------------------------------------------
def gemm_exact(qx, qw) -> np.ndarray:
    """acc[t, o] = sum_k dec(qx[t, k]) * dec(qw[k, o]), exact, float64."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    T, Ci = qx.shape
    Ci2, Co = qw.shape
    assert Ci == Ci2
    acc = np.empty((T, Co), dtype=np.float64)
    lib().orc_gemm_exact(_ptr(qx), Ci, _ptr(qw), Co, T, Ci, Co, _ptr(acc))
    return acc


def gemm_exact_i64(qx, qw) -> np.ndarray:
    """The same sum in integer units of 2^-18 (int64)."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    T, Ci = qx.shape
    Co = qw.shape[1]
    acc = np.empty((T, Co), dtype=np.int64)
    lib().orc_gemm_exact_i64(_ptr(qx), Ci, _ptr(qw), Co, T, Ci, Co, _ptr(acc))
    return acc


def gemm_exact_sampled(qx, qw, rows, cols) -> np.ndarray:
    """Exact sums for the outputs (rows[i], cols[i]) only."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    T, Ci = qx.shape
    Co = qw.shape[1]
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < T)
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < Co)
    acc = np.empty(rows.size, dtype=np.float64)
    lib().orc_gemm_exact_sampled(_ptr(qx), Ci, _ptr(qw), Co, Ci, _ptr(rows),
                                 _ptr(cols), rows.size, _ptr(acc))
    return acc


def apply_scales(acc, dx, dw) -> np.ndarray:
    """ref[t, o] = acc[t, o] * dx[t] * dw[o] in double."""
    acc = _c(acc, np.float64)
    dx = _c(dx, np.float32)
    dw = _c(dw, np.float32)
    T, Co = acc.shape
    ref = np.empty((T, Co), dtype=np.float64)
    lib().orc_apply_scales(_ptr(acc), T, Co, _ptr(dx), _ptr(dw), _ptr(ref))
    return ref


def apply_scales_sampled(acc, rows, cols, dx, dw) -> np.ndarray:
    acc = _c(acc, np.float64)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    dx = _c(dx, np.float32)
    dw = _c(dw, np.float32)
    ref = np.empty(rows.size, dtype=np.float64)
    lib().orc_apply_scales_sampled(_ptr(acc), _ptr(rows), _ptr(cols), rows.size,
                                   _ptr(dx), _ptr(dw), _ptr(ref))
    return ref


def gemm_dequant_first(qx, dx, qw, dw) -> np.ndarray:
    """sum_k (dec(qx)*dx[t]) * (dec(qw)*dw[o]) -- scales applied before the sum."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    dx = _c(dx, np.float32)
    dw = _c(dw, np.float32)
    T, Ci = qx.shape
    Co = qw.shape[1]
    out = np.empty((T, Co), dtype=np.float64)
    lib().orc_gemm_dequant_first(_ptr(qx), Ci, _ptr(dx), _ptr(qw), Co, _ptr(dw),
                                 T, Ci, Co, _ptr(out))
    return out


def ptpc_linear(x, w):
    """The whole path on the CPU: quantize X and W, contract exactly, scale.

    Returns a dict with codes, scales, the exact sum, the double reference
    output and its bf16 rounding.
    """
    qx, dx = quant_act(x)
    qw, dw = quant_weight(w)
    acc = gemm_exact(qx, qw)
    ref = apply_scales(acc, dx, dw)
    return dict(qx=qx, dx=dx, qw=qw, dw=dw, acc=acc, ref=ref,
                out_bf16=bf16_from_double(ref))
