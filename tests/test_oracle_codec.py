"""Pins for the oracle's E4M3 codec and bf16 rounding (CPU only).

The codec is checked against things other than itself:
  * the OCP OFP8 v1.0 E4M3 table (tests/golden/e4m3_ocp_values.txt);
  * PyTorch's own float8_e4m3fn decoding and casting (a library routine);
  * a brute-force nearest-value search over the 254 finite code values,
    using values decoded by PyTorch, not by the oracle.
"""
import numpy as np
import pytest
import torch

from conftest import read_golden

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_force_encode(f32):
    """Nearest finite E4M3 value (ties -> even code), saturating, sign kept."""
    f32 = np.asarray(f32, dtype=np.float32)
    vals = torch_decode(FINITE)                    # PyTorch's decoding
    pos = FINITE[vals > 0]
    posv = vals[vals > 0]
    mags = np.concatenate([[0.0], posv])           # 0 and the 126 positive values
    codes = np.concatenate([[0], pos]).astype(np.uint8)
    order = np.argsort(mags)
    mags, codes = mags[order], codes[order]
    a = np.abs(f32.astype(np.float64))
    out = np.empty(f32.shape, dtype=np.uint8)
    step = 1 << 16
    af, of = a.reshape(-1), out.reshape(-1)
    for i in range(0, af.size, step):
        blk = af[i:i + step, None]
        d = np.abs(blk - mags[None, :])
        best = d.min(axis=1, keepdims=True)
        tie = d == best
        # among equally near candidates take the even code (mantissa LSB 0)
        even = tie & ((codes[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
        c = codes[pick]
        c = np.where(blk[:, 0] >= 448.0, np.uint8(0x7E), c)   # saturate
        of[i:i + step] = c
    return out | np.where(np.signbit(f32), np.uint8(0x80), np.uint8(0))


def all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32)
    exp = (b >> 7) & 0xFF
    b = b[exp != 0xFF]
    return (b << 16).view(np.float32)


def test_decode_matches_ocp_table(orc):
    g = read_golden("e4m3_ocp_values.txt")
    for code_s, vals in g.items():
        code = int(code_s, 16)
        want = float(vals[0][0])
        got = orc.e4m3_decode(np.array([code]))[0]
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), code_s


def test_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    want = torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(want[m]))
    assert set(np.flatnonzero(np.isnan(got))) == {0x7F, 0xFF}


def test_encode_roundtrip_every_finite_code(orc):
    vals = torch_decode(FINITE).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), FINITE)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8, 2.0 ** -3, 0.7, 3.0, 2.0 ** 6,
                                   2.0 ** -120])
def test_encode_brute_force_all_bf16(orc, scale):
    f = all_bf16_finite().astype(np.float64) * scale
    f = f[np.abs(f) < 3e38].astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(f), brute_force_encode(f))


def test_encode_brute_force_midpoints(orc):
    v = np.sort(torch_decode(FINITE[torch_decode(FINITE) >= 0]))
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)       # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (v[1:] + v[:-1]) / 2)
    f = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(np.inf)),
                        np.float32([448, 464, 463.99997, 464.00003, 1e6, 0, 2.0 ** -10,
                                    2.0 ** -149])])
    f = np.concatenate([f, -f])
    assert np.array_equal(orc.e4m3_encode(f), brute_force_encode(f))


def test_encode_random_fp32_brute_force(orc):
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(orc.e4m3_encode(f), brute_force_encode(f))


def test_encode_matches_torch_cast_below_464(orc):
    """PyTorch's float32 -> float8_e4m3fn cast rounds to nearest even; it does
    not saturate (NaN from 464 up), so compare only where |v| < 464, which
    covers every quotient x / (amax/448)."""
    rng = np.random.default_rng(5)
    f = np.concatenate([all_bf16_finite(),
                        rng.standard_normal(500_000).astype(np.float32) * 50,
                        (rng.random(500_000) * 464).astype(np.float32)])
    f = f[np.abs(f) < 464]
    want = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(f), want)


def test_encode_sign_and_zero(orc):
    f = np.float32([0.0, -0.0, -1e-30, 1e-30, -2.0 ** -11, 2.0 ** -11, -448, -1e9, 1e9])
    assert list(orc.e4m3_encode(f)) == [0x00, 0x80, 0x80, 0x00, 0x80, 0x00, 0xFE, 0xFE, 0x7E]


def test_bf16_from_double_matches_torch_on_fp32_values(orc):
    """For doubles that are fp32 values a single rounding to bf16 is what
    PyTorch's float32 -> bfloat16 cast does (round to nearest even)."""
    rng = np.random.default_rng(3)
    u = rng.integers(0, 1 << 32, size=300_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    # include exact ties: bf16 value + half a bf16 ulp
    ties = ((rng.integers(0, 1 << 16, 20_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < 3e38)]
    f = np.concatenate([f, ties])
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_from_double(f.astype(np.float64)), want)


def test_bf16_from_double_is_nearest(orc):
    """Generic doubles: the result brackets the value and is the nearer of
    the two neighbouring bf16 values (ties to even)."""
    rng = np.random.default_rng(4)
    v = rng.standard_normal(100_000) * np.exp(rng.uniform(-60, 60, 100_000))
    r = orc.bf16_from_double(v)
    rv = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    step_up = ((r.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    step_dn = ((r.astype(np.uint32) - 1) << 16).view(np.float32).astype(np.float64)
    err = np.abs(v - rv)
    assert np.all(err <= np.abs(v - step_up))
    assert np.all(err <= np.abs(v - step_dn))
