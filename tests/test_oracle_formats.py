"""Pins for the oracle's FP8 decode/encode against what the format definitions fix.

None of these re-types the oracle's formula: the encode is checked against a
brute-force nearest-value search over the decoded code table, against the
published constants (tests/golden/fp8_format_constants.json), and against
PyTorch's own CPU FP8 conversion for in-range values.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2, decode, decode_table, encode

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp8_format_constants.json")
FMTS = [E4M3, E5M2]


def _gold():
    with open(GOLD) as f:
        return json.load(f)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_published_constants(fmt):
    g = _gold()[fmt.name]
    assert fmt.bias == g["exponent_bias"]
    assert fmt.max == g["max_normal"]
    t = decode_table(fmt)
    finite = t[np.isfinite(t)]
    assert finite.max() == g["max_normal"]
    pos = finite[finite > 0]
    assert pos.min() == g["min_subnormal"]
    assert decode(1 << fmt.man_bits, fmt) == g["min_normal"]
    assert decode((1 << fmt.man_bits) - 1, fmt) == g["max_subnormal"]
    nan_mags = [c for c in range(128) if np.isnan(decode(c, fmt))]
    assert nan_mags == g["nan_magnitude_codes"]
    if g["infinities"]:
        assert decode(g["inf_magnitude_code"], fmt) == float("inf")
        assert decode(0x80 | g["inf_magnitude_code"], fmt) == float("-inf")
    else:
        assert not np.isinf(t).any()


def test_closed_form_maxima():
    # 1.75 * 2^8 and 1.75 * 2^15
    assert E4M3.max == 1.75 * 2 ** 8 == 448.0
    assert E5M2.max == 1.75 * 2 ** 15 == 57344.0
    assert decode(0x7E, E4M3) == 448.0 and decode(0xFE, E4M3) == -448.0
    assert decode(0x7B, E5M2) == 57344.0 and decode(0xFB, E5M2) == -57344.0
    assert decode(0x38, E4M3) == 1.0 and decode(0x3C, E5M2) == 1.0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_roundtrip_all_256_codes(fmt):
    t = decode_table(fmt)
    codes = encode(t.astype(np.float32), fmt)
    for c in range(256):
        v = t[c]
        if np.isnan(v):
            assert np.isnan(decode(int(codes[c]), fmt)), c
        elif np.isinf(v):
            # saturating cast: infinities map to +-max
            assert codes[c] == (0x80 if v < 0 else 0) | fmt.max_code
        else:
            assert codes[c] == c, (c, v, codes[c])


def _brute_nearest(x: float, fmt) -> int:
    """Nearest finite code by exhaustive search; ties go to the even code.

    Saturation: |x| >= max gives +-max.  Sign is kept for zero results."""
    if np.isnan(x):
        return -1
    neg = np.signbit(x)
    a = abs(x)
    if a >= fmt.max:
        return (0x80 if neg else 0) | fmt.max_code
    best = None
    for c in range(fmt.max_code + 1):
        v = decode(c, fmt)
        d = abs(Fraction(a) - Fraction(v))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return (0x80 if neg else 0) | best[1]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_rne_at_every_midpoint(fmt):
    t = decode_table(fmt)
    vals = sorted(set(float(v) for v in t[: fmt.max_code + 1]))
    probes = []
    for u, v in zip(vals[:-1], vals[1:]):
        mid = np.float32((u + v) / 2)
        assert float(mid) == (u + v) / 2  # midpoints are fp32-representable
        probes += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]
    probes = np.array(probes, dtype=np.float32)
    probes = np.concatenate([probes, -probes])
    got = encode(probes, fmt)
    for x, c in zip(probes, got):
        assert c == _brute_nearest(float(x), fmt), (float(x), c)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_random_values_brute_force(fmt):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(300).astype(np.float32) * np.float32(fmt.max / 8),
        (rng.standard_normal(300) * 2.0 ** rng.integers(-20, 4, 300)).astype(np.float32),
    ])
    got = encode(x, fmt)
    for xi, c in zip(x, got):
        assert c == _brute_nearest(float(xi), fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_saturation(fmt):
    fmax = np.finfo(np.float32).max
    x = np.array([fmt.max, np.nextafter(np.float32(fmt.max), np.float32(np.inf)), 2 * fmt.max,
                  1e30, fmax, np.inf], dtype=np.float32)
    assert (encode(x, fmt) == fmt.max_code).all()
    assert (encode(-x, fmt) == (0x80 | fmt.max_code)).all()
    # just below max stays max; the next lower code is not reached by rounding
    assert encode(np.float32(fmt.max) * np.float32(0.999), fmt) == fmt.max_code


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_nan_and_signed_zero(fmt):
    c = encode(np.array([np.nan, -np.nan], dtype=np.float32), fmt)
    for ci in c:
        assert np.isnan(decode(int(ci), fmt))
    assert encode(np.float32(0.0), fmt) == 0x00
    assert encode(np.float32(-0.0), fmt) == 0x80
    assert encode(np.float32(-1e-30), fmt) == 0x80
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    assert encode(tiny, fmt) == 0x00 and encode(-tiny, fmt) == 0x80


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_monotone(fmt):
    rng = np.random.default_rng(11)
    x = np.sort(np.concatenate([
        rng.uniform(-fmt.max * 1.2, fmt.max * 1.2, 20000),
        rng.standard_normal(20000) * 0.01]).astype(np.float32))
    v = decode_table(fmt)[encode(x, fmt)]
    assert (np.diff(v) >= 0).all()


@pytest.mark.parametrize("fmt,tdt", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)],
                         ids=["E4M3", "E5M2"])
def test_matches_torch_cpu_cast_in_range(fmt, tdt):
    rng = np.random.default_rng(3)
    t = decode_table(fmt)
    vals = np.array(sorted(set(float(v) for v in t[: fmt.max_code + 1])))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        (rng.standard_normal(50000) * fmt.max / 16).astype(np.float32),
        (rng.standard_normal(50000) * 2.0 ** rng.integers(-24, 0, 50000)).astype(np.float32),
    ])
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < fmt.max]
    ref = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    got = encode(x, fmt)
    np.testing.assert_array_equal(got, ref)
