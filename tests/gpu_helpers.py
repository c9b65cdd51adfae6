"""Shared helpers for the GPU parity tests (host side only)."""
import os

import numpy as np
import torch

import oracle

# bf16-output acceptance: max |gpu - ref| <= 2^-7 max |ref| and relative L2
# error <= 4e-3 against the oracle's double-precision reference.
MAX_REL = 2.0 ** -7
L2_REL = 4e-3


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nan_filled(T, Co):
    """A bf16 [T, Co] output buffer on the GPU holding NaN in every element."""
    return torch.full((T, Co), float("nan"), dtype=torch.bfloat16, device="cuda")


def no_nan(t: torch.Tensor, what: str):
    """Every element of a GPU output was written (none is still NaN)."""
    n = int(torch.isnan(t).sum().item())
    assert n == 0, f"{what}: {n} outputs never written (still NaN)"


def check_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str):
    """The acceptance bar on a set of outputs (full or sampled)."""
    got = bf16_bits_to_f64(gpu_bits)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    max_err = float(err.max()) if err.size else 0.0
    assert max_err <= MAX_REL * scale, f"{what}: max err {max_err} > 2^-7 * {scale}"
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / nrm if nrm > 0 else 0.0
    log = os.environ.get("PTPC_PARITY_LOG")
    if log:
        # one line per checked output set: the figures the bar is applied to
        with open(log, "a") as f:
            f.write(f"{what}\t{got.size}\t{max_err / scale if scale else 0.0:.3e}\t{rel:.3e}\n")
    assert rel <= L2_REL, f"{what}: rel L2 {rel} > {L2_REL}"
    return max_err, scale


def sample_indices(T, Co, n, seed):
    """Outputs to check at full size: random (t, o) pairs plus whole first /
    last rows and columns chunks (tile edges)."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(0, T, n), np.full(min(Co, 512), T - 1), np.zeros(min(Co, 512), np.int64)]
    cols = [rng.integers(0, Co, n), np.arange(min(Co, 512)), Co - 1 - np.arange(min(Co, 512))]
    k = min(T, 256)
    rows += [np.arange(k), T - 1 - np.arange(k)]
    cols += [np.full(k, Co - 1), np.zeros(k, np.int64)]
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def oracle_sampled_ref(qx, dx, qw, dw, rows, cols):
    acc = oracle.gemm_exact_sampled(qx, qw, rows, cols)
    return oracle.apply_scales_sampled(acc, rows, cols, dx, dw)


def packed_byte_index(Ci, Co):
    """Byte offset in the packed weight of the code of w[k][o], for every
    (k, o) with k < Kp, from the layout include/ptpc.h documents:
    block (g, s) = (o // 16, k // 64) at (g * Kp/64 + s) * 1024; unit
    u = 4 * (o % 16) + (c ^ ((o % 16) // 4 % 4)) with c = (k % 64) // 16;
    byte k % 16 of the unit.  Returns an int64 array [Kp, Co]."""
    Kp = (Ci + 127) // 128 * 128
    k = np.arange(Kp, dtype=np.int64)[:, None]
    o = np.arange(Co, dtype=np.int64)[None, :]
    row = o % 16
    c = (k % 64) // 16
    u = 4 * row + (c ^ ((row // 4) % 4))
    return ((o // 16) * (Kp // 64) + k // 64) * 1024 + u * 16 + k % 16
