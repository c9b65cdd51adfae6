"""Seeded synthetic inputs for the PTPC-FP8 linear layers.

This module only draws numbers: it holds none of the quantization or GEMM
arithmetic, and it is the one piece of code that both the CPU oracle's tests
and the GPU library's tests / benchmark use, so that both sides see the same
bf16 bits.

Shapes follow Llama-3.1-8B / 70B linear layers; the value structure follows
the outlier model of vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD
ROCm", §The outlier problem and §PTPC: a precision-targeted scheme -- outliers
sit in the same few channels for every token, channel magnitudes vary a lot
within a token and stay stable across tokens, weights are near-uniform.

Recipe (every draw from ``numpy.random.Generator(PCG64)``, float32 draws
scaled in float32, then rounded to bf16 with round-to-nearest-even):

  tiny          X [16 x 256] ~ N(0,1), channels {3,77,130,201} x 50;
                W [256 x 512] ~ N(0, 0.02^2).
  8b_qkv_decode X [32 x 4096] ~ N(0,1); 1% of channels (41, drawn without
                replacement) each times a fixed factor ~ U[20,100]; one drawn
                row set to zero.  W [4096 x 6144] ~ N(0, 0.02^2).
  8b_gate_up    X [2048 x 4096], same outlier model (no zero row);
                W [4096 x 28672] ~ N(0, 0.02^2).
  70b_down      X [4096 x 28672] = |z1| * silu(z2), z ~ N(0,1) i.i.d.;
                1% of channels (287) x 50.  W [28672 x 8192] ~ N(0, 0.01^2).
  70b_sweep     layer in {qkv 8192->10240, o 8192->8192,
                gate_up 8192->57344, down 28672->8192}, T in {1,16,128,1024,
                8192}: X[t,k] = s[t,k] * m[k], s ~ Student-t(3) i.i.d.,
                m[k] = exp(1.5 n_k), n_k ~ N(0,1) fixed per channel; for T >= 16
                one drawn row is zero and another drawn row gets one entry set
                to a value drawn from U[500, 5e4] (sign drawn); for T = 1 the
                single row gets that planted entry.  W ~ N(0, 0.01^2) per layer.

  GPU draws     (timing only, no oracle side: the benchmark's per-shape
                lines for the 70B layers at 1024 / 8192 tokens and the 8B
                gate_up layer) the same value structure drawn on the GPU by
                torch's seeded Philox generator: Student-t(3) as z / sqrt(chi2_3 / 3)
                from four normals, times exp(1.5 n_k) per channel, one zero row
                and one planted value in [500, 5e4]; or N(0,1) with 1% outlier
                channels times U[20,100]; weights N(0, sigma^2).

  70b model load  (timing only, no oracle side) every linear weight of the
                80 decoder layers, qkv / o / gate_up / down shapes as above,
                W ~ N(0, 0.01^2) drawn in bf16 on the GPU by torch's seeded
                Philox generator (seed = 1000 * layer + index).

Draw order per call: X base, outlier channels, outlier factors, special
rows, then W from its own stream.  X and W use separate generators
(``default_rng([seed, tag, ...])``) so a layer's W is the same for every T.
"""
from dataclasses import dataclass

import numpy as np

SWEEP_LAYERS = {
    "qkv": (8192, 10240),
    "o": (8192, 8192),
    "gate_up": (8192, 57344),
    "down": (28672, 8192),
}
SWEEP_T = (1, 16, 128, 1024, 8192)

_CHUNK = 1 << 22  # elements per generation chunk (bounds float64 temporaries)


@dataclass(frozen=True)
class Shape:
    name: str
    T: int
    Ci: int
    Co: int


CONFIGS = {
    "tiny": Shape("tiny", 16, 256, 512),
    "8b_qkv_decode": Shape("8b_qkv_decode", 32, 4096, 6144),
    "8b_gate_up": Shape("8b_gate_up", 2048, 4096, 28672),
    "70b_down": Shape("70b_down", 4096, 28672, 8192),
}


def sweep_shape(layer: str, T: int) -> Shape:
    Ci, Co = SWEEP_LAYERS[layer]
    return Shape(f"70b_sweep_{layer}_T{T}", T, Ci, Co)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng, rows, cols, sigma):
    """rows x cols of N(0, sigma^2), drawn row-chunk by row-chunk."""
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            z *= np.float32(sigma)
        out[r0:r1] = f32_to_bf16_bits(z)
    return out


def _outlier_normal_x(rng, T, Ci, n_out, fac_lo, fac_hi, zero_row):
    x = rng.standard_normal((T, Ci), dtype=np.float32)
    ch = rng.choice(Ci, size=n_out, replace=False)
    fac = rng.uniform(fac_lo, fac_hi, size=n_out).astype(np.float32)
    x[:, ch] *= fac
    if zero_row:
        x[rng.integers(T), :] = 0.0
    return f32_to_bf16_bits(x)


def _silu_skew_x(rng, T, Ci, n_out, factor):
    out = np.empty((T, Ci), dtype=np.uint16)
    step = max(1, _CHUNK // Ci)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        z1 = rng.standard_normal((r1 - r0, Ci), dtype=np.float32)
        z2 = rng.standard_normal((r1 - r0, Ci), dtype=np.float32)
        out[r0:r1] = f32_to_bf16_bits(np.abs(z1) * (z2 / (np.float32(1) + np.exp(-z2))))
    ch = rng.choice(Ci, size=n_out, replace=False)
    vals = bf16_bits_to_f32(out[:, ch]) * np.float32(factor)
    out[:, ch] = f32_to_bf16_bits(vals)
    return out


def _student_lognormal_x(rng, T, Ci):
    m = np.exp(1.5 * rng.standard_normal(Ci)).astype(np.float32)
    out = np.empty((T, Ci), dtype=np.uint16)
    step = max(1, _CHUNK // Ci)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        s = rng.standard_t(3, size=(r1 - r0, Ci)).astype(np.float32)
        out[r0:r1] = f32_to_bf16_bits(s * m)
    if T >= 16:
        zr, pr = rng.choice(T, size=2, replace=False)
        out[zr, :] = 0
    else:
        pr = 0
    col = rng.integers(Ci)
    val = np.float32(rng.uniform(500.0, 5.0e4) * (1 if rng.random() < 0.5 else -1))
    out[pr, col] = f32_to_bf16_bits(np.array([val], dtype=np.float32))[0]
    return out


def make(name: str, seed: int = 0, T: int = None, layer: str = None):
    """Return (shape, X bf16 bits [T x Ci], W bf16 bits [Ci x Co])."""
    if name == "70b_sweep":
        shape = sweep_shape(layer, T)
        li = list(SWEEP_LAYERS).index(layer)
        rx = np.random.default_rng([seed, 5, li, T])
        rw = np.random.default_rng([seed, 5, li, 1 << 20])
        x = _student_lognormal_x(rx, shape.T, shape.Ci)
        w = _normal_bf16(rw, shape.Ci, shape.Co, 0.01)
        return shape, x, w
    shape = CONFIGS[name]
    if T is not None:
        shape = Shape(shape.name, T, shape.Ci, shape.Co)
    tag = list(CONFIGS).index(name) + 1
    rx = np.random.default_rng([seed, tag, 0])
    rw = np.random.default_rng([seed, tag, 1])
    if name == "tiny":
        x = rx.standard_normal((shape.T, shape.Ci), dtype=np.float32)
        x[:, [3, 77, 130, 201]] *= np.float32(50)
        x = f32_to_bf16_bits(x)
        w = _normal_bf16(rw, shape.Ci, shape.Co, 0.02)
    elif name in ("8b_qkv_decode", "8b_gate_up"):
        n_out = int(round(0.01 * shape.Ci))
        x = _outlier_normal_x(rx, shape.T, shape.Ci, n_out, 20.0, 100.0,
                              zero_row=(name == "8b_qkv_decode"))
        w = _normal_bf16(rw, shape.Ci, shape.Co, 0.02)
    elif name == "70b_down":
        n_out = int(round(0.01 * shape.Ci))
        x = _silu_skew_x(rx, shape.T, shape.Ci, n_out, 50.0)
        w = _normal_bf16(rw, shape.Ci, shape.Co, 0.01)
    else:
        raise KeyError(name)
    return shape, x, w


def random_bf16(rng, rows, cols, sigma=1.0):
    """Plain N(0, sigma^2) bf16 matrix (for ad-hoc shapes in tests)."""
    return _normal_bf16(rng, rows, cols, sigma)


LLAMA70B_LAYERS = 80


def device_weight(layer: int, index: int, Ci: int, Co: int, sigma: float, device):
    """One synthetic bf16 weight [Ci x Co] drawn directly on `device` (torch's
    seeded Philox generator), for load-time measurements at model scale where
    host generation and transfer of ~140 GB would dominate."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(1000 * layer + index)
    return torch.empty((Ci, Co), device=device, dtype=torch.bfloat16).normal_(0.0, sigma,
                                                                             generator=g)


def device_activation(kind: str, T: int, Ci: int, seed: int, device):
    """Synthetic bf16 activations [T x Ci] drawn on `device` (timing only):
    kind "student_lognormal" (the 70B layer sweep's structure) or
    "outlier_normal" (the 8B layers' structure)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = dict(device=device, dtype=torch.float32)
    if kind == "student_lognormal":
        m = torch.exp(1.5 * torch.randn(Ci, generator=g, **f32))
        x = torch.empty((T, Ci), device=device, dtype=torch.bfloat16)
        step = max(1, (1 << 24) // Ci)
        for r0 in range(0, T, step):
            r1 = min(T, r0 + step)
            z = torch.randn((r1 - r0, Ci), generator=g, **f32)
            chi2 = torch.zeros_like(z)
            for _ in range(3):
                chi2.add_(torch.randn((r1 - r0, Ci), generator=g, **f32).square_())
            x[r0:r1] = (z / torch.sqrt(chi2 / 3.0) * m).to(torch.bfloat16)
        if T >= 16:
            x[T // 3] = 0
        x[T // 2, Ci // 5] = 12345.0
        return x
    if kind == "outlier_normal":
        x = torch.randn((T, Ci), generator=g, **f32)
        n_out = max(1, int(round(0.01 * Ci)))
        ch = torch.randperm(Ci, generator=g, device=device)[:n_out]
        fac = 20.0 + 80.0 * torch.rand(n_out, generator=g, **f32)
        x[:, ch] *= fac
        return x.to(torch.bfloat16)
    raise KeyError(kind)
