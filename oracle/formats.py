"""FP8 formats E4M3 and E5M2: bit-field decode and saturating round-to-nearest-even encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [FP8-intro] section "FP8 Training について" says FP8 is an 8-bit float
format with a narrow dynamic range; [FP8-intro] section "Transformer Engine の
使い方" (code comment on ``Format.HYBRID``) fixes E4M3 for the forward pass and
E5M2 for the backward pass; [TE-summary] section "導入とリソース" points to the
original FP8 paper (arXiv:2209.05433), whose definitions are used here for the
bit fields:

  E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits.  No infinities; the only
        NaN magnitude is S.1111.111.  Largest finite S.1111.110 = 1.75 * 2^8 = 448.
  E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-like: S.11111.00 is
        infinity, S.11111.{01,10,11} are NaN.  Largest finite 1.75 * 2^15 = 57344.

Readings taken where the pages are silent:
  * rounding is round-to-nearest, ties to even;
  * the cast saturates: finite values at or above the largest finite magnitude,
    and infinities, map to +-max;
  * NaN maps to the NaN code 0x7F (with the sign bit of the input);
  * subnormals are produced and the sign of zero is kept (-0 -> 0x80).

Pins (tests/test_oracle_formats.py): exhaustive 256-code round trip, closed-form
maxima and minimum subnormals, brute-force nearest-code search at every
midpoint, saturation, monotonicity, and agreement with PyTorch's own CPU FP8
conversion for in-range values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class FP8Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    has_inf: bool  # E5M2 has infinities; E4M3 (the "FN" variant) does not

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal number (1 - bias)."""
        return 1 - self.bias

    @property
    def max_code(self) -> int:
        """Magnitude code of the largest finite value."""
        top_exp = (1 << self.exp_bits) - 1
        if self.has_inf:
            # top exponent field reserved for Inf/NaN; largest finite uses top-1
            return ((top_exp - 1) << self.man_bits) | ((1 << self.man_bits) - 1)
        # E4M3: top exponent field is usable, only mantissa all-ones is NaN
        return (top_exp << self.man_bits) | ((1 << self.man_bits) - 2)

    @property
    def max(self) -> float:
        return _decode_magnitude(self.max_code, self)

    @property
    def nan_code(self) -> int:
        return 0x7F


E4M3 = FP8Format("E4M3", 4, 3, 7, False)
E5M2 = FP8Format("E5M2", 5, 2, 15, True)


def fp8_format(name: str) -> FP8Format:
    return {"E4M3": E4M3, "E5M2": E5M2}[name.upper()]


def _decode_magnitude(mag: int, fmt: FP8Format) -> float:
    """Value of a 7-bit magnitude code, from the bit-field definition."""
    e_field = mag >> fmt.man_bits
    m_field = mag & ((1 << fmt.man_bits) - 1)
    top_exp = (1 << fmt.exp_bits) - 1
    if fmt.has_inf and e_field == top_exp:
        return float("inf") if m_field == 0 else float("nan")
    if not fmt.has_inf and e_field == top_exp and m_field == (1 << fmt.man_bits) - 1:
        return float("nan")
    if e_field == 0:  # subnormal: 0.m * 2^emin
        return m_field * 2.0 ** (fmt.emin - fmt.man_bits)
    return (1.0 + m_field / (1 << fmt.man_bits)) * 2.0 ** (e_field - fmt.bias)


def decode(code: int, fmt: FP8Format) -> float:
    """Value of one FP8 code (exact as a Python float)."""
    code = int(code) & 0xFF
    v = _decode_magnitude(code & 0x7F, fmt)
    return -v if code & 0x80 else v


def decode_table(fmt: FP8Format) -> np.ndarray:
    """All 256 code values as float64 (exact)."""
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(v, fmt: FP8Format) -> np.ndarray:
    """Saturating round-to-nearest-even encode of fp32 values to FP8 codes.

    ``v`` is converted to float32 first (the value being encoded is an fp32
    number), then widened exactly to float64 for the arithmetic.

    For a finite |v| below the largest finite value, with
    e = max(floor(log2 |v|), emin) and quantum q = 2^(e - mbits), the encoded
    magnitude is r*q where r = round_half_even(|v| / q); the magnitude code is
    ((e + bias - 1) << mbits) + r, which covers subnormals (e = emin gives
    code = r) and a round-up into the next binade (r = 2^(mbits+1)).
    """
    v32 = np.asarray(v, dtype=np.float32)
    x = v32.astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    is_nan = np.isnan(x)
    sat = (~is_nan) & (a >= fmt.max)
    a_fin = np.where(is_nan | sat, 0.0, a)

    _, e = np.frexp(a_fin)  # a = frac * 2^e with frac in [0.5, 1)  ->  floor(log2 a) = e - 1
    e = np.maximum(e.astype(np.int64) - 1, fmt.emin)
    q = np.ldexp(1.0, (e - fmt.man_bits).astype(np.int32))
    r = np.rint(a_fin / q).astype(np.int64)  # np.rint rounds half to even; a_fin/q is exact
    mag = ((e + fmt.bias - 1) << fmt.man_bits) + r
    mag = np.where(a_fin == 0.0, 0, mag)
    mag = np.where(sat, fmt.max_code, mag)
    mag = np.where(is_nan, fmt.nan_code, mag)
    code = mag | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)
