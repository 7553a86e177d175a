"""MXFP4: E2M1 elements with one E8M0 power-of-two scale per 32 elements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[LP-opt] "実モデルにおける結果の解釈" compares the FP4 tensor-core GEMMs with
MXFP8 on the same shapes (FP4 1.46-1.66x faster on the large GEMMs); its NVFP4
recipe needs E4M3 scales per 16 elements, which a matrix core with E8M0 scales
per 32 elements does not apply.  The FP4 variant built here is therefore MXFP4 (OCP Microscaling
Formats v1.0), the block format of the MXFP8 recipe ([TE-summary] "主な機能")
with 4-bit elements.  Readings:

  * E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
    0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6; no infinity or NaN codes;
  * the element cast rounds to nearest, ties to the even mantissa, and
    saturates at +-6; the sign of zero is kept;
  * block scale as in MXFP8: e = floor(log2(amax)) - 2 (6 = 1.5 * 2^2), clamped
    to [-127, 127], code e + 127, 127 for an all-zero block; elements
    satRNE(x * 2^-e); an infinite amax has log2 = +inf, so e = 127 (code 254),
    its infinities saturate to +-6 and the block's finite elements go to 0;
  * a block holding a NaN gets the NaN scale code 255 (E2M1 has no NaN, so the
    scale carries it) and its elements are cast with e = 0, NaN to +0;
  * two codes per byte, element 2i in the low nibble, 2i + 1 in the high one.

The recipe steps around this quantizer (Hadamard transform, stochastic rounding, 2D
weight blocks) are in fp4_recipe.py.

Pins (tests/test_oracle_mxfp4.py): the 16-code table from its bit fields, the
round trip of every code, every midpoint tie, saturation and monotonicity of
the encoder, block scales of closed-form blocks, the packing, and the MXFP4
GEMM against a Python loop and against plain products at unit scales.
"""

from __future__ import annotations

import numpy as np

from .gemm import _epilogue
from .quantize import e8m0_to_float

BLOCK = 32
_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode_table() -> np.ndarray:
    """value of each 4-bit code (bit 3 sign, bits 2-1 exponent, bit 0 mantissa), float64."""
    out = np.empty(16)
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        out[c] = s * (m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))
    return out


def e2m1_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even E2M1 codes (uint8 0..15) of float values."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a = np.where(np.isnan(a), 0.0, np.minimum(a, 6.0))
    d = np.abs(a[..., None] - _MAGS)                  # distance to each magnitude
    best = np.min(d, axis=-1, keepdims=True)
    tie_even = np.where(d == best, (np.arange(8) & 1) * 2 + np.arange(8) * 1e-9, np.inf)
    idx = np.argmin(tie_even, axis=-1)                # nearest, the even mantissa on a tie
    sign = np.where(np.signbit(x) & ~np.isnan(x), 8, 0)
    return (idx + sign).astype(np.uint8)


def pack(codes) -> np.ndarray:
    """[R, C] codes -> [R, C/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def block_exponent(xb):
    """The scale rule for blocks along the last axis of xb (float64): (e, e8m0 codes).
    e = floor(log2 amax) - 2 clamped to [-127, 127]; 0 for an all-zero block; 127 for an
    infinite amax; a block holding a NaN gets e = 0 and code 255."""
    nan = np.any(np.isnan(xb), axis=-1)
    am = np.max(np.where(np.isnan(xb), 0.0, np.abs(xb)), axis=-1)
    fin = np.isfinite(am)
    _, fe = np.frexp(np.where((am > 0) & fin, am, 1.0))
    e = np.where(am > 0, fe.astype(np.int64) - 1 - 2, 0)
    e = np.where(fin, e, 127)                          # log2 of an infinite amax is +inf
    e = np.where(nan, 0, np.clip(e, -127, 127))
    return e, np.where(nan, 255, e + 127).astype(np.uint8)


def mxfp4_quantize(x):
    """(packed codes uint8 [R, C/2], e8m0 uint8 [R, C/32]) of the rows of x (fp32 values)."""
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    if C % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    xb = x32.reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    e, scale_codes = block_exponent(xb)
    scaled = np.ldexp(xb, (-e)[:, :, None].astype(np.int32))
    return pack(e2m1_encode(scaled).reshape(R, C)), scale_codes


def dequantize(packed, e8m0) -> np.ndarray:
    """float64 values of an MXFP4 tensor (NaN where the scale code is 255)."""
    v = e2m1_decode_table()[unpack(packed)]
    s = np.where(np.asarray(e8m0) == 255, np.nan, e8m0_to_float(np.where(np.asarray(e8m0) == 255, 127, e8m0)))
    return v * np.repeat(s, BLOCK, axis=1)


def gemm_mxfp4(a_packed, a_e8m0, b_packed, b_e8m0, bias=None, out: str = "bf16") -> np.ndarray:
    """D = A B^T with A, B MXFP4 [M, K], [N, K] (packed): every product and every
    power-of-two scaling is exact in float64; the sum is rounded once to fp32."""
    acc = (dequantize(a_packed, a_e8m0) @ dequantize(b_packed, b_e8m0).T).astype(np.float32)
    return _epilogue(acc, bias, out)
