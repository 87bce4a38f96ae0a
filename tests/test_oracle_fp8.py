"""Pins of the oracle's E4M3 codec against things other than itself:
the format's published special values (golden file), torch's independent
float8_e4m3fn conversion (a library routine), exhaustive midpoint rounding,
saturation, and the analytic round-trip bound."""
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), float(val)))
    return rows


def test_golden_points():
    rows = _golden()
    assert len(rows) >= 10
    for code, val in rows:
        d = fp8.DECODE_TABLE[code]
        if np.isnan(val):
            assert np.isnan(d), hex(code)
        else:
            assert d == val and np.signbit(d) == np.signbit(val), (hex(code), d, val)
            if code not in (0x80,):
                assert fp8.encode(np.float32(val))[()] == code, hex(code)


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8.DECODE_TABLE
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(mine))
    assert np.array_equal(ref[~nan_ref], mine[~nan_ref])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(mine[~nan_ref]))
    assert nan_ref.sum() == 2  # exactly 0x7F and 0xFF


def _torch_encode(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_values():
    v = fp8.DECODE_TABLE
    return np.unique(np.abs(v[np.isfinite(v)]))  # 0 .. 448, 127 values


def test_encode_matches_torch_on_codes_midpoints_and_neighbours():
    vals = _finite_values()
    mids = (vals[:-1] + vals[1:]) / 2.0  # exactly representable in float32
    pts = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    allp = np.concatenate([pts, up, dn])
    allp = allp[allp < 464.0]  # torch maps >= 464 to NaN; saturation is checked below
    allp = np.concatenate([allp, -allp])
    assert np.array_equal(fp8.encode(allp), _torch_encode(allp))


def test_midpoints_round_to_even_mantissa():
    vals = _finite_values()
    codes = fp8.encode(vals.astype(np.float32))
    mids = ((vals[:-1] + vals[1:]) / 2.0).astype(np.float32)
    got = fp8.encode(mids)
    lo, hi = codes[:-1], codes[1:]
    expect = np.where((lo & 1) == 0, lo, hi)
    assert np.array_equal(got, expect)


def test_encode_matches_torch_random():
    rng = np.random.default_rng(123)
    n = 1_000_000
    mag = np.exp2(rng.uniform(-14, np.log2(463.9), n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    assert np.array_equal(fp8.encode(x), _torch_encode(x))
    # raw float32 bit patterns below 464 in magnitude, including subnormals
    bits = rng.integers(0, 0x43E80000, n, dtype=np.uint32)
    y = bits.view(np.float32)
    y = np.where(rng.random(n) < 0.5, -y, y).astype(np.float32)
    assert np.array_equal(fp8.encode(y), _torch_encode(y))


def test_roundtrip_of_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    fin = np.isfinite(fp8.DECODE_TABLE)
    back = fp8.encode(fp8.DECODE_TABLE_F32[fin])
    assert np.array_equal(back, codes[fin])


def test_saturation_inf_and_nan():
    big = np.array([448.0, 448.01, 463.99, 464.0, 480.0, 1e4, 3.4e38, np.inf], dtype=np.float32)
    assert np.all(fp8.encode(big) == 0x7E)
    assert np.all(fp8.encode(-big) == 0xFE)
    n = fp8.encode(np.array([np.nan, -np.nan], dtype=np.float32))
    assert (n[0] & 0x7F) == 0x7F and (n[1] & 0x7F) == 0x7F


@pytest.mark.parametrize("scale", [1.0, 0.0171875, 3.25e-3, 7.0])
def test_roundtrip_error_bound(scale):
    """|x_hat - x| <= 2^-4 |x| in the normal range, <= 2^-10 * sigma in the
    subnormal range (half the code spacing), for |x / sigma| <= 448."""
    rng = np.random.default_rng(7)
    n = 1_000_000
    u = np.exp2(rng.uniform(-12, np.log2(448.0), n)) * rng.choice([-1.0, 1.0], n)
    x = (u * scale).astype(np.float32)
    s = np.float32(scale)
    xh = fp8.dequantize(fp8.quantize(x, s), s, np.float64)
    err = np.abs(xh - x.astype(np.float64))
    r = np.abs(x.astype(np.float64) / s)
    normal = r >= 2.0 ** -6
    # float32 division adds at most a relative 2^-24; allow that slack.
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 2e-7) + 1e-30)
    assert np.all(err[~normal] <= 2.0 ** -10 * scale * (1 + 1e-6) + 1e-30)
