"""Pins for oracle/formats.py: code tables and round-to-nearest-even encoders.

Each test pins the oracle to something other than itself: values the pages
print (tests/golden/fp8_ranges.txt), the closed-form E2M1 value set, brute
force over every code and every midpoint, and torch's own float8 casts.
"""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()[:2]
            out[k] = float(v)
    return out


def test_fp8_maxima_match_pages():
    g = _golden("fp8_ranges.txt")
    assert F.E5M2.max_value == g["e5m2_max"] == 57344.0
    # the page's E4M3 figure is the FNUZ (bias 8) maximum ...
    assert F.e4m3fnuz_max() == g["e4m3_max_printed"] == 240.0
    # ... while the format used here (float8_e4m3fn, bias 7) tops out at 448
    assert F.E4M3.max_value == 448.0
    assert F.E4M3.max_code == 0x7E and F.E5M2.max_code == 0x7B


def test_e2m1_value_set_and_max():
    # OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; max 6.0 (E2M1_MAX)
    assert list(F.E2M1.values[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.E2M1.values[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert F.E2M1.max_value == 6.0


def test_special_codes():
    assert np.isnan(F.E4M3.values[0x7F]) and np.isnan(F.E4M3.values[0xFF])
    assert np.sum(np.isnan(F.E4M3.values)) == 2          # E4M3FN: no Inf
    assert F.E5M2.values[0x7C] == np.inf and F.E5M2.values[0xFC] == -np.inf
    assert np.sum(np.isnan(F.E5M2.values)) == 6
    assert F.E4M3.values[0x01] == 2.0 ** -9                # smallest subnormal
    assert F.E5M2.values[0x01] == 2.0 ** -16
    assert F.e8m0_value(127) == 1.0 and F.e8m0_value(254) == 2.0 ** 127
    assert F.e8m0_value(0) == 2.0 ** -127 and np.isnan(F.e8m0_value(255))


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2, F.E2M1])
def test_decode_encode_identity_all_codes(fmt):
    codes = np.arange(1 << fmt.bits)
    vals = F.decode(codes, fmt)
    finite = np.isfinite(vals)
    back = F.encode(vals[finite], fmt)
    assert np.array_equal(back, codes[finite].astype(np.uint8))


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2, F.E2M1])
def test_midpoints_ties_to_even_and_neighbours(fmt):
    mags = fmt.values[: fmt.max_code + 1]
    for c in range(fmt.max_code):
        lo, hi = mags[c], mags[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        for sgn, sbit in ((1.0, 0), (-1.0, fmt.sign_bit)):
            assert F.encode(sgn * mid, fmt) == even | sbit
            assert F.encode(sgn * np.nextafter(mid, 0), fmt) == c | sbit
            assert F.encode(sgn * np.nextafter(mid, np.inf), fmt) == (c + 1) | sbit


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2, F.E2M1])
def test_saturation_and_signed_zero(fmt):
    mx = fmt.max_value
    big = np.array([mx, mx * 1.01, mx * 1.5, mx * 1e6, 3e38])
    assert np.all(F.encode(big, fmt) == fmt.max_code)
    assert np.all(F.encode(-big, fmt) == fmt.max_code | fmt.sign_bit)
    assert F.encode(0.0, fmt) == 0
    assert F.encode(-0.0, fmt) == fmt.sign_bit
    assert F.encode(1e-300, fmt) == 0 and F.encode(-1e-300, fmt) == fmt.sign_bit
    with pytest.raises(ValueError):
        F.encode(np.nan, fmt)


@pytest.mark.parametrize("fmt,tdtype", [(F.E4M3, torch.float8_e4m3fn), (F.E5M2, torch.float8_e5m2)])
def test_encode_matches_torch_float8_cast(fmt, tdtype):
    """Library cross-check: torch's CPU float8 cast (RNE) on in-range fp32 values."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= fmt.max_value)]
    # add every midpoint and every exact value
    mags = fmt.values[: fmt.max_code + 1]
    extra = np.concatenate([mags, (mags[1:] + mags[:-1]) / 2]).astype(np.float32)
    x = np.concatenate([x, extra, -extra])
    ref = torch.from_numpy(x).to(tdtype).view(torch.uint8).numpy()
    got = F.encode(x.astype(np.float64), fmt)
    assert np.array_equal(got, ref)


def test_e2m1_encode_matches_brute_force_nearest():
    """Brute force on E2M1: distance to all 8 magnitudes, ties to the even code."""
    mags = F.E2M1.values[:8]
    for x in np.linspace(-8, 8, 16001):
        a = abs(x)
        d = np.abs(mags - a)
        cands = np.flatnonzero(d == d.min())
        c = int(cands[0]) if len(cands) == 1 else [int(k) for k in cands if k % 2 == 0][0]
        if a >= 6:
            c = 7
        want = c | (8 if np.signbit(x) else 0)
        assert F.encode(x, F.E2M1) == want, x
