"""GPU parity: libptpc (through its C ABI) against the CPU oracle.

FP8 codes and scales must be bit-identical; bf16 GEMM outputs must satisfy
max |gpu - ref| <= 2^-7 max |ref| and relative L2 <= 4e-3 against the
oracle's exact-sum reference; the fused and two-step GEMMs must agree
bit-for-bit.  Shapes: the five workload families at full size (GEMM outputs
sampled where the oracle would take minutes), plus ragged and degenerate
shapes checked in full.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity_shapes as ps
import workloads
from gpu_helpers import (bits_to_dev, check_close, dev_to_bits, nan_filled, no_nan,
                         oracle_sampled_ref, packed_byte_index, sample_indices)

pytestmark = pytest.mark.gpu

sg = None


@pytest.fixture(scope="module", autouse=True)
def gpu_lib():
    global sg
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_gemm_amd
    sg = scaled_gemm_amd
    sg.lib()
    yield


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_path(x_bits, w_bits):
    """Quantize X and W and run both GEMMs on the GPU; return host copies."""
    x = bits_to_dev(x_bits)
    w = bits_to_dev(w_bits)
    T, Co = x_bits.shape[0], w_bits.shape[1]
    qx, dx = sg.quant_act(x)
    pw = sg.quant_weight(w)
    # every output starts as NaN: a tile the kernels skip cannot pass
    out = sg.gemm(qx, dx, pw, out=nan_filled(T, Co))
    out2 = sg.gemm_unfused(qx, dx, pw, out=nan_filled(T, Co))
    ws3 = nan_filled(T, Co)
    out3 = sg.gemm_unfused_bf16(qx, dx, pw, out=nan_filled(T, Co), workspace=ws3)
    qw = sg.unpack_weight(pw)
    torch.cuda.synchronize()
    for o, what in ((out, "fused"), (out2, "two-step"), (out3, "bf16 two-step"),
                    (ws3, "bf16 intermediate")):
        no_nan(o, what)
    return dict(qx=qx.cpu().numpy(), dx=dx.cpu().numpy(), qw=qw.cpu().numpy(),
                dw=pw.dw.cpu().numpy(), out=dev_to_bits(out), out2=dev_to_bits(out2),
                out3=dev_to_bits(out3), ws3=dev_to_bits(ws3), packed=pw.data.cpu().numpy())


def check_bf16_two_step(g, ref, what, rows=None, cols=None):
    """The bf16-intermediate two-step form: within the bar of the exact
    reference, and its step 2 is exactly bf16((ws * dx[t]) * dw[o]) in fp32."""
    out3, ws3 = g["out3"], g["ws3"]
    T, Co = ws3.shape
    if rows is None:
        check_close(out3, ref, f"{what} bf16 two-step")
        w32 = workloads.bf16_bits_to_f32(ws3)
        want = workloads.f32_to_bf16_bits((w32 * g["dx"][:, None]) * g["dw"][None, :])
        assert np.array_equal(out3, want), f"{what}: bf16 two-step step 2"
    else:
        check_close(out3[rows, cols], ref, f"{what} bf16 two-step (sampled)")
        w32 = workloads.bf16_bits_to_f32(ws3[rows, cols])
        want = workloads.f32_to_bf16_bits((w32 * g["dx"][rows]) * g["dw"][cols])
        assert np.array_equal(out3[rows, cols], want), f"{what}: bf16 two-step step 2"


def check_quant(g, x_bits, w_bits, what):
    qx, dx = oracle.quant_act(x_bits)
    assert np.array_equal(g["dx"], dx), f"{what}: dx differs"
    bad = np.argwhere(g["qx"] != qx)
    assert bad.size == 0, f"{what}: {len(bad)} activation codes differ, first {bad[:5].tolist()}"
    qw, dw = oracle.quant_weight(w_bits)
    assert np.array_equal(g["dw"], dw), f"{what}: dw differs"
    bad = np.argwhere(g["qw"] != qw)
    assert bad.size == 0, f"{what}: {len(bad)} weight codes differ, first {bad[:5].tolist()}"
    Ci, Co = w_bits.shape
    if Ci * Co <= (1 << 26):
        # the documented packed layout, read directly (not via unpack_weight)
        idx = packed_byte_index(Ci, Co)
        packed = g["packed"]
        assert packed.size == idx.size, f"{what}: packed size"
        assert np.array_equal(packed[idx[:Ci]], qw), f"{what}: packed layout"
        assert np.all(packed[idx[Ci:]] == 0), f"{what}: K padding not zero"
    return qx, dx, qw, dw


# ---------------------------------------------------------------------------
# small and ragged shapes: whole outputs against the full oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,seed", ps.FULL_SEEDS)
def test_full_parity_other_seeds(name, seed):
    note(f"full parity {name} seed={seed}")
    _, x, w = workloads.make(name, seed=seed)
    g = run_path(x, w)
    qx, dx, qw, dw = check_quant(g, x, w, f"{name} seed {seed}")
    ref = oracle.apply_scales(oracle.gemm_exact(qx, qw), dx, dw)
    check_close(g["out"], ref, f"{name} seed {seed} fused")
    assert np.array_equal(g["out"], g["out2"]), "fused and two-step differ"


def ragged_inputs(T, Ci, Co):
    """Seeded inputs of any shape: N(0,1) activations with every (Ci/7)-th
    channel scaled by 60 and a zero row, N(0, 0.02^2) weights with a zero
    column."""
    rng = np.random.default_rng(T * 7 + Ci)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, :: max(1, Ci // 7)] = workloads.f32_to_bf16_bits(
        workloads.bf16_bits_to_f32(x[:, :: max(1, Ci // 7)]) * np.float32(60))
    if T > 2:
        x[1] = 0
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    if Co > 16:
        w[:, 5] = 0
    return x, w


@pytest.mark.parametrize("name,T,Ci,Co", ps.FULL_CASES)
def test_full_parity(name, T, Ci, Co):
    note(f"full parity {name} T={T} Ci={Ci} Co={Co}")
    if name == "ragged":
        x, w = ragged_inputs(T, Ci, Co)
    else:
        _, x, w = workloads.make(name)
    g = run_path(x, w)
    qx, dx, qw, dw = check_quant(g, x, w, name)
    ref = oracle.apply_scales(oracle.gemm_exact(qx, qw), dx, dw)
    check_close(g["out"], ref, f"{name} fused")
    assert np.array_equal(g["out"], g["out2"]), "fused and two-step differ"
    check_bf16_two_step(g, ref, name)


# ---------------------------------------------------------------------------
# full-size workloads: codes/scales in full, GEMM on sampled outputs
# ---------------------------------------------------------------------------
def sampled_case(x, w, what, seed):
    g = run_path(x, w)
    qx, dx, qw, dw = check_quant(g, x, w, what)
    T, Co = x.shape[0], w.shape[1]
    rows, cols = sample_indices(T, Co, 3000, seed)
    ref = oracle_sampled_ref(qx, dx, qw, dw, rows, cols)
    out = g["out"].reshape(T, Co)
    check_close(out[rows, cols], ref, f"{what} fused (sampled)")
    assert np.array_equal(g["out"], g["out2"]), f"{what}: fused and two-step differ"
    check_bf16_two_step(g, ref, what, rows, cols)
    return g


@pytest.mark.parametrize("T,Ci,Co", ps.TILE_CASES)
def test_tile_shape_parity(T, Ci, Co):
    note(f"tile-shape parity T={T} Ci={Ci} Co={Co}")
    x, w = ragged_inputs(T, Ci, Co)
    sampled_case(x, w, f"T={T} Ci={Ci} Co={Co}", seed=T + Ci)


@pytest.mark.parametrize("name", ps.CONFIG_CASES)
def test_config_parity(name):
    note(f"config parity {name}")
    shape, x, w = workloads.make(name)
    sampled_case(x, w, name, seed=1)


@pytest.mark.parametrize("layer,T", ps.EXTRA_SWEEP_CASES)
def test_extra_sweep_shape_parity(layer, T):
    note(f"70b {layer} T={T} (sampled)")
    shape, x, w = workloads.make("70b_sweep", T=T, layer=layer)
    sampled_case(x, w, shape.name, seed=T)


@pytest.mark.parametrize("layer", list(workloads.SWEEP_LAYERS))
def test_sweep_parity(layer):
    """One 70B layer shape for every T; the weight is quantized once."""
    w = None
    for T in workloads.SWEEP_T:
        shape, x, w_t = workloads.make("70b_sweep", T=T, layer=layer)
        if w is None:
            w = w_t
            note(f"70b sweep {layer}: weight {w.shape}")
            pw = sg.quant_weight(bits_to_dev(w))
            qw_o, dw_o = oracle.quant_weight(w)
            assert np.array_equal(pw.dw.cpu().numpy(), dw_o)
            assert np.array_equal(sg.unpack_weight(pw).cpu().numpy(), qw_o)
        else:
            assert np.array_equal(w_t, w)     # same weight stream for every T
        note(f"70b sweep {layer} T={T}")
        xd = bits_to_dev(x)
        qx, dx = sg.quant_act(xd)
        o1 = sg.gemm(qx, dx, pw, out=nan_filled(T, shape.Co))
        o2 = sg.gemm_unfused(qx, dx, pw, out=nan_filled(T, shape.Co))
        no_nan(o1, f"{shape.name} fused")
        no_nan(o2, f"{shape.name} two-step")
        out = dev_to_bits(o1).reshape(T, -1)
        out2 = dev_to_bits(o2).reshape(T, -1)
        del o1, o2
        qx_o, dx_o = oracle.quant_act(x)
        assert np.array_equal(dx.cpu().numpy(), dx_o)
        assert np.array_equal(qx.cpu().numpy(), qx_o)
        rows, cols = sample_indices(T, shape.Co, 2000, seed=T)
        ref = oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols)
        check_close(out[rows, cols], ref, f"{shape.name} (sampled)")
        assert np.array_equal(out, out2), f"{shape.name}: fused and two-step differ"
        del xd, qx, dx


# ---------------------------------------------------------------------------
# exhaustive per-element check of the activation quantizer
# ---------------------------------------------------------------------------
def test_quant_act_exhaustive_pairs():
    """Every (x, amax) pair of bf16 values with |x| <= amax, both signs: one
    row per (amax, sign) holding amax and every smaller magnitude.  The code
    of an element depends only on x and its row's amax, so this covers every
    input the quantizer can see (rows of various lengths exercise each
    launch shape)."""
    amax_all = np.arange(1, 0x7F80, dtype=np.int32)       # positive finite bf16
    buckets = ps.EXHAUSTIVE_CI
    total = 0
    lo = 0
    for Ci in buckets:
        hi = min(Ci - 1, amax_all[-1] + 1)                 # rows need a + 2 <= Ci
        sel = amax_all[(amax_all >= lo) & (amax_all < hi)]
        lo = hi
        if sel.size == 0:
            continue
        step = max(1, (1 << 25) // Ci)
        for s0 in range(0, sel.size, step):
            a = sel[s0:s0 + step].astype(np.int32)
            idx = np.arange(Ci, dtype=np.int32)[None, :] - 1
            pos = np.where(idx <= a[:, None], idx, 0)
            pos[:, 0] = a
            neg = np.where(idx <= a[:, None], idx | 0x8000, 0)
            neg[:, 0] = a | 0x8000
            x = np.concatenate([pos, neg]).astype(np.uint16)
            note(f"exhaustive quant Ci={Ci} rows={x.shape[0]} amax {a[0]:#06x}..{a[-1]:#06x}")
            qg, dg = sg.quant_act(bits_to_dev(x))
            qo, do = oracle.quant_act(x)
            assert np.array_equal(dg.cpu().numpy(), do)
            qg = qg.cpu().numpy()
            bad = np.argwhere(qg != qo)
            assert bad.size == 0, (f"{len(bad)} codes differ; first (row, col, x, gpu, oracle): " +
                                   str([(int(r), int(c), hex(x[r, c]), hex(qg[r, c]), hex(qo[r, c]))
                                        for r, c in bad[:5]]))
            total += x.shape[0]
    assert total == 2 * amax_all.size


@pytest.mark.parametrize("T,Ci", ps.LONG_ROW_CASES)
def test_quant_act_long_rows(T, Ci):
    """Long rows (32 vectors per thread in registers, and rows longer than
    one workgroup holds: amax pass, then a second read): codes and scales
    bit-exact, with each row's largest magnitude placed in a different part
    of the row, the last row's in the last 16-byte vector."""
    note(f"long-row quant_act T={T} Ci={Ci}")
    rng = np.random.default_rng(Ci + T)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    for t in range(T):
        # rows 0, 3, 6 (the last): inside the last 16-byte vector
        k = Ci - 8 + t % 8 if t % 3 == 0 else int(rng.integers(0, Ci))
        x[t, k] = workloads.f32_to_bf16_bits(np.array([(-1) ** t * (50.0 + t)], np.float32))[0]
    qbuf = torch.full((T, Ci), 0xAB, dtype=torch.uint8, device="cuda")
    qx, dx = sg.quant_act(bits_to_dev(x), qx=qbuf)
    qo, do = oracle.quant_act(x)
    assert np.array_equal(dx.cpu().numpy(), do)
    assert np.array_equal(qx.cpu().numpy(), qo)
    big = np.abs(workloads.bf16_bits_to_f32(x)).argmax(axis=1)
    assert big[T - 1] >= Ci - 8 and np.all((qo[np.arange(T), big] & 0x7F) == 0x7E)


def test_quant_weight_column_extremes():
    """Weight columns with subnormal, tiny, huge and ordinary amax, each
    holding a sweep of smaller magnitudes of both signs."""
    Ci = 4096
    amaxes = np.array([0x0001, 0x0005, 0x007F, 0x0080, 0x00FF, 0x0C00, 0x1234, 0x3F80,
                       0x3F81, 0x43E0, 0x43E1, 0x5000, 0x7000, 0x7F7F, 0x2000, 0x6543], np.int64)
    rng = np.random.default_rng(7)
    cols = []
    for a in amaxes:
        mags = rng.integers(0, a + 1, Ci)
        mags[rng.integers(Ci)] = a
        signs = rng.integers(0, 2, Ci) << 15
        cols.append((mags | signs).astype(np.uint16))
    w = np.stack(cols, axis=1)
    w = np.concatenate([w, np.zeros((Ci, 16), np.uint16)], axis=1)   # plus 16 zero columns
    pw = sg.quant_weight(bits_to_dev(w))
    qw = sg.unpack_weight(pw).cpu().numpy()
    qo, do = oracle.quant_weight(w)
    assert np.array_equal(pw.dw.cpu().numpy(), do)
    assert np.array_equal(qw, qo)


# ---------------------------------------------------------------------------
# degenerate and layout cases
# ---------------------------------------------------------------------------
def test_empty_and_zero_extents():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    qx, dx = sg.quant_act(x)
    assert qx.shape == (0, 256) and dx.shape == (0,)
    # Ci == 0: every row scale is 1, and the GEMM output is zero
    x0 = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    qx0, dx0 = sg.quant_act(x0)
    torch.cuda.synchronize()
    assert torch.all(dx0 == 1.0)
    w0 = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    pw0 = sg.PackedWeight(torch.empty(0, dtype=torch.uint8, device="cuda"),
                          torch.empty(32, dtype=torch.float32, device="cuda"), 0, 32)
    sg.quant_weight(w0, out=pw0)
    out = sg.gemm(qx0, dx0, pw0)
    torch.cuda.synchronize()
    assert torch.all(pw0.dw == 1.0)
    assert torch.all(out.float() == 0.0)
    # Co == 0
    w1 = torch.empty((64, 0), dtype=torch.bfloat16, device="cuda")
    pw1 = sg.quant_weight(w1)
    q1, d1 = sg.quant_act(torch.ones((3, 64), dtype=torch.bfloat16, device="cuda"))
    assert sg.gemm(q1, d1, pw1).shape == (3, 0)


@pytest.mark.parametrize("T,Ci,Co", ps.PITCHED_CASES)
def test_pitched_inputs_and_outputs(T, Ci, Co):
    """Row pitches larger than the extents (views into wider buffers): the
    K-split 64x64 tiles, the 64x128 tiles at 256+ tokens and the 128-byte-step
    tiled kernel."""
    rng = np.random.default_rng(12)
    xb = workloads.random_bf16(rng, T, Ci + 40, 1.0)
    wb = workloads.random_bf16(rng, Ci, Co + 24, 0.02)
    xd = bits_to_dev(xb)[:, :Ci]
    wd = bits_to_dev(wb)[:, :Co]
    qbuf = torch.full((T, Ci + 48), 0xAB, dtype=torch.uint8, device="cuda")
    qx, dx = sg.quant_act(xd, qx=qbuf[:, :Ci])
    pw = sg.quant_weight(wd)
    obuf = torch.zeros((T, Co + 32), dtype=torch.bfloat16, device="cuda")
    sg.gemm(qx, dx, pw, out=obuf[:, :Co])
    torch.cuda.synchronize()
    x = np.ascontiguousarray(xb[:, :Ci])
    w = np.ascontiguousarray(wb[:, :Co])
    qo, do = oracle.quant_act(x)
    assert np.array_equal(qbuf[:, :Ci].cpu().numpy(), qo)
    assert np.all(qbuf[:, Ci:].cpu().numpy() == 0xAB)          # pitch padding untouched
    qwo, dwo = oracle.quant_weight(w)
    ref = oracle.apply_scales(oracle.gemm_exact(qo, qwo), do, dwo)
    o = dev_to_bits(obuf)
    check_close(o[:, :Co], ref, "pitched")
    assert np.all(o[:, Co:] == 0)


@pytest.mark.parametrize("reps", [6, 12])
def test_power_of_two_row_scaling_and_permutation(reps):
    """Scaling a token by 2^k scales its output by exactly 2^k; permuting
    tokens permutes output rows bit-for-bit."""
    _, x, w = workloads.make("tiny")
    x = np.concatenate([x] * reps)                     # 96 or 192 rows
    rng = np.random.default_rng(0)
    pw = sg.quant_weight(bits_to_dev(w))
    base = dev_to_bits(sg.linear(bits_to_dev(x), pw))
    xs = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x) * np.float32(8))
    scaled = dev_to_bits(sg.linear(bits_to_dev(xs), pw))
    b = (base.astype(np.uint32) << 16).view(np.float32)
    s = (scaled.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(s, b * np.float32(8))
    perm = rng.permutation(x.shape[0])
    permuted = dev_to_bits(sg.linear(bits_to_dev(np.ascontiguousarray(x[perm])), pw))
    assert np.array_equal(permuted, base[perm])
    # a weight column times 2^k: same codes, its scale and output column times 2^k
    ws = workloads.bf16_bits_to_f32(w).copy()
    ws[:, 5] *= np.float32(4)
    ws[:, 17] *= np.float32(0.25)
    pw2 = sg.quant_weight(bits_to_dev(workloads.f32_to_bf16_bits(ws)))
    col = dev_to_bits(sg.linear(bits_to_dev(x), pw2))
    c = (col.astype(np.uint32) << 16).view(np.float32)
    want = b.copy()
    want[:, 5] *= np.float32(4)
    want[:, 17] *= np.float32(0.25)
    assert np.array_equal(c, want)


# ---------------------------------------------------------------------------
# split-K GEMM (ptpc_gemm_ws) for token counts with too few output tiles
# ---------------------------------------------------------------------------
def test_gemm_ws_split_k_ragged():
    """K cut into ranges (here 4, the last one holding the K tail), rows and
    columns ragged: whole output against the oracle, deterministic across
    calls, and the workspace contents do not matter."""
    T, Ci, Co = 200, 4112, 400
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need == 4 * 4 * T * Co
    rng = np.random.default_rng(31)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, ::97] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, ::97]) * np.float32(30))
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")     # NaN-pattern garbage
    a = dev_to_bits(sg.gemm_ws(qx, dx, pw, workspace=ws))
    b = dev_to_bits(sg.gemm_ws(qx, dx, pw))
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    ref = oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o)
    check_close(a, ref, "split-K ragged")
    assert np.array_equal(a, b), "split-K not deterministic"


def test_gemm_ws_split_k_256_ragged():
    """From 256 tokens on with K >= 12288 the workspace form runs 256x256
    tiles of the 16x16x128 kernel over K ranges: here 8 ranges of 13 steps
    of 128 bytes, the last one 6 steps ending in a 16-byte K tail, rows
    ragged (300 = 256 + 44) and columns ragged (528 = 2 x 256 + 16).  Whole
    output against the oracle, deterministic, workspace contents ignored."""
    T, Ci, Co = 300, 12304, 528
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need == 8 * 4 * T * Co
    note(f"split-K 256x256 ragged T={T} Ci={Ci} Co={Co}")
    rng = np.random.default_rng(37)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, ::89] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, ::89]) * np.float32(30))
    x[:, -3:] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, -3:]) * np.float32(20))
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")     # NaN-pattern garbage
    o = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co), workspace=ws)
    no_nan(o, "split-K 256x256 ragged")
    a = dev_to_bits(o)
    b = dev_to_bits(sg.gemm_ws(qx, dx, pw))
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    ref = oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o)
    check_close(a, ref, "split-K 256x256 ragged")
    assert np.array_equal(a, b), "split-K not deterministic"


def test_gemm_ws_split_k_256_max_k():
    """The 256x256 split at the contract's K limit (Ci = 2^17 - 16): 8 K
    ranges of 128 steps, the last ending 16 bytes short of a whole step;
    rows 260 = 256 + 4, columns 144 (one ragged column tile).  Whole output
    against the oracle."""
    T, Ci, Co = 260, (1 << 17) - 16, 144
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need == 8 * 4 * T * Co
    note(f"split-K 256x256 max K T={T} Ci={Ci} Co={Co}")
    rng = np.random.default_rng(41)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, -5:] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, -5:]) * np.float32(25))
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    o = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co))
    no_nan(o, "split-K 256x256 max K")
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    ref = oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o)
    check_close(dev_to_bits(o), ref, "split-K 256x256 max K")


def test_gemm_ws_split_k_256_rows_129_255():
    """At 129..255 tokens with long K the workspace form runs one 256-row
    tile per weight slab (256x256 tiles, rows past T out of range): 200
    tokens, K 16400 (8 ranges of 17 steps of 128 bytes, the last 10 steps
    with a 16-byte tail), 528 columns.  Whole output against the oracle; then
    the 70B QKV (where ptpc_gemm runs 128x128 tiles: 6 ranges) and down
    (8 ranges) layers at 200 tokens, sampled, within a bf16 ulp-scale of
    ptpc_gemm."""
    T, Ci, Co = 200, 16400, 528
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need == 8 * 4 * T * Co
    note(f"split-K 256x256 at {T} tokens: Ci={Ci} Co={Co}")
    rng = np.random.default_rng(43)
    x = workloads.random_bf16(rng, T, Ci, 1.0)
    x[:, ::71] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x[:, ::71]) * np.float32(30))
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    qx, dx = sg.quant_act(bits_to_dev(x))
    pw = sg.quant_weight(bits_to_dev(w))
    o = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co))
    no_nan(o, "split-K 256x256 at 200 tokens")
    qx_o, dx_o = oracle.quant_act(x)
    qw_o, dw_o = oracle.quant_weight(w)
    ref = oracle.apply_scales(oracle.gemm_exact(qx_o, qw_o), dx_o, dw_o)
    check_close(dev_to_bits(o), ref, "split-K 256x256 at 200 tokens")
    del qx, dx, pw
    for layer, S in (("qkv", 6), ("down", 8)):
        shape, x, w = workloads.make("70b_sweep", T=200, layer=layer)
        assert sg.gemm_workspace_bytes(200, shape.Ci, shape.Co) == S * 4 * 200 * shape.Co
        note(f"split-K 70b {layer} T=200 S={S}")
        qx, dx = sg.quant_act(bits_to_dev(x))
        pw = sg.quant_weight(bits_to_dev(w))
        o = sg.gemm_ws(qx, dx, pw, out=nan_filled(200, shape.Co))
        no_nan(o, f"70b {layer} T=200 split-K")
        out = dev_to_bits(o)
        plain = dev_to_bits(sg.gemm(qx, dx, pw))
        qx_o, dx_o = oracle.quant_act(x)
        qw_o, dw_o = oracle.quant_weight(w)
        rows, cols = sample_indices(200, shape.Co, 3000, seed=9)
        ref = oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols)
        check_close(out[rows, cols], ref, f"70b {layer} T=200 split-K (sampled)")
        d = np.abs(bf16_f32(out) - bf16_f32(plain))
        assert d.max() <= 2.0 ** -7 * np.abs(bf16_f32(plain)).max()
        del qx, dx, pw


def test_gemm_ws_long_k_256_plus():
    """The 70B down projection (K = 28672) at 256 tokens (32 tiles of
    256x256, 8 K ranges) and 1024 tokens (128 tiles, 2 ranges) through
    ptpc_gemm_ws: every output written, sampled outputs against the oracle,
    within a bf16 ulp of ptpc_gemm (another fp32 summation order)."""
    shape, x, w = workloads.make("70b_down", T=1024)
    pw = sg.quant_weight(bits_to_dev(w))
    qw_o, dw_o = oracle.quant_weight(w)
    for T, S in ((256, 8), (1024, 2)):
        xs = np.ascontiguousarray(x[:T])
        assert sg.gemm_workspace_bytes(T, shape.Ci, shape.Co) == (
            S * 4 * T * shape.Co if S > 2 else fixup_ws_bytes(T, shape.Co))
        note(f"split-K 70b down T={T} S={S}")
        qx, dx = sg.quant_act(bits_to_dev(xs))
        o = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, shape.Co))
        no_nan(o, f"70b down T={T} split-K")
        out = dev_to_bits(o)
        plain = dev_to_bits(sg.gemm(qx, dx, pw))
        qx_o, dx_o = oracle.quant_act(xs)
        rows, cols = sample_indices(T, shape.Co, 3000, seed=7)
        ref = oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols)
        check_close(out[rows, cols], ref, f"70b down T={T} split-K (sampled)")
        d = np.abs(bf16_f32(out) - bf16_f32(plain))
        assert d.max() <= 2.0 ** -7 * np.abs(bf16_f32(plain)).max()
        del qx, dx


def fixup_ws_bytes(T, Co):
    """Workspace of a two-range split over 256x256 tiles: an fp32 slot of
    256x256 per tile, then a 4-word record per tile."""
    return ((T + 255) // 256) * ((Co + 255) // 256) * (4 * 256 * 256 + 16)


def fixup_records(ws, T, Co):
    """The per-tile records [tickets taken, published flag, 0, 0] a two-range
    call leaves in its workspace."""
    n = ((T + 255) // 256) * ((Co + 255) // 256)
    rec = ws[n * 4 * 256 * 256:n * (4 * 256 * 256 + 16)].cpu().numpy()
    return rec.view(np.uint32).reshape(n, 4)


def test_gemm_ws_two_range_fixup():
    """Two K ranges over 256x256 tiles, joined inside the GEMM kernel (the
    range that finishes second adds the first's published sums): 300 tokens
    (rows ragged: 256 + 44), K 16400 (65 + 64 steps of 128 bytes, a 16-byte
    tail), 10768 columns (42 x 256 + 16): 86 tiles, 172 workgroups.  The
    workspace starts as garbage (record words included); every output is
    written, sampled outputs match the oracle, the whole output is within a
    bf16 ulp-scale of ptpc_gemm, every tile's record shows both tickets taken
    and the sums published, and a second call with other activations over
    the same workspace gives that call's result, bit-identical to a call on
    a fresh workspace."""
    T, Ci, Co = 300, 16400, 10768
    need = sg.gemm_workspace_bytes(T, Ci, Co)
    assert need == fixup_ws_bytes(T, Co) == 86 * (4 * 256 * 256 + 16)
    note(f"two-range fix-up T={T} Ci={Ci} Co={Co}")
    rng = np.random.default_rng(47)
    w = workloads.random_bf16(rng, Ci, Co, 0.02)
    pw = sg.quant_weight(bits_to_dev(w))
    qw_o, dw_o = oracle.quant_weight(w)
    del w
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")     # NaN-pattern garbage
    ws[86 * 4 * 256 * 256:] = 0x5A                                          # garbage records
    for call, seed in ((1, 48), (2, 49)):
        x = workloads.random_bf16(np.random.default_rng(seed), T, Ci, 1.0)
        x[:, ::83] = workloads.f32_to_bf16_bits(
            workloads.bf16_bits_to_f32(x[:, ::83]) * np.float32(30))
        x[:, -4:] = workloads.f32_to_bf16_bits(
            workloads.bf16_bits_to_f32(x[:, -4:]) * np.float32(20))
        qx, dx = sg.quant_act(bits_to_dev(x))
        o = sg.gemm_ws(qx, dx, pw, out=nan_filled(T, Co), workspace=ws)
        no_nan(o, f"two-range fix-up call {call}")
        out = dev_to_bits(o)
        rec = fixup_records(ws, T, Co)
        assert np.all(rec[:, 0] == 2) and np.all(rec[:, 1] == 1), f"records after call {call}"
        fresh = dev_to_bits(sg.gemm_ws(qx, dx, pw))
        assert np.array_equal(out, fresh), f"call {call} depends on the workspace it found"
        plain = dev_to_bits(sg.gemm(qx, dx, pw))
        d = np.abs(bf16_f32(out) - bf16_f32(plain))
        assert d.max() <= 2.0 ** -7 * np.abs(bf16_f32(plain)).max()
        qx_o, dx_o = oracle.quant_act(x)
        rows, cols = sample_indices(T, Co, 4000, seed=call)
        ref = oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols)
        check_close(out[rows, cols], ref, f"two-range fix-up call {call} (sampled)")
        del qx, dx, x


def test_gemm_ws_sweep_t128():
    """The 70B layers at 128 tokens through ptpc_gemm_ws (QKV: 3 K ranges;
    down, K = 28672: 4; O, whose 64x64 tiles split K inside the workgroup,
    and gate_up: no split -> bit-identical to ptpc_gemm)."""
    for layer in workloads.SWEEP_LAYERS:
        shape, x, w = workloads.make("70b_sweep", T=128, layer=layer)
        note(f"split-K 70b {layer} T=128")
        qx, dx = sg.quant_act(bits_to_dev(x))
        pw = sg.quant_weight(bits_to_dev(w))
        o = sg.gemm_ws(qx, dx, pw, out=nan_filled(128, shape.Co))
        no_nan(o, f"{shape.name} split-K")
        out = dev_to_bits(o)
        plain = dev_to_bits(sg.gemm(qx, dx, pw))
        if sg.gemm_workspace_bytes(128, shape.Ci, shape.Co) == 0:
            assert np.array_equal(out, plain)
            continue
        qx_o, dx_o = oracle.quant_act(x)
        qw_o, dw_o = oracle.quant_weight(w)
        rows, cols = sample_indices(128, shape.Co, 3000, seed=3)
        ref = oracle_sampled_ref(qx_o, dx_o, qw_o, dw_o, rows, cols)
        check_close(out[rows, cols], ref, f"{shape.name} split-K (sampled)")
        # another fp32 summation order than ptpc_gemm: equal up to a bf16 ulp
        d = np.abs(bf16_f32(out) - bf16_f32(plain))
        assert d.max() <= 2.0 ** -7 * np.abs(bf16_f32(plain)).max()
        del qx, dx, pw


def bf16_f32(b):
    return workloads.bf16_bits_to_f32(b).astype(np.float64)
