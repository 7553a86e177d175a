"""The FP4 recipe's extra steps around the MXFP4 quantizer: random Hadamard transform of
the Wgrad inputs, stochastic rounding of gradients, 2D block scaling of weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[LP-opt] "実モデルにおける結果の解釈" (diagnosis "GEMM の速度向上 >> トレーニングの速度向
上") names these as the FP4 recipe's overhead beyond the GEMM: a random Hadamard
transform on the inputs of Wgrad, stochastic rounding of gradients, 2D block scaling of
weights, and an extra memory pass for a per-tensor amax.  The pages give no formula for
any of them; the readings (the plainest standard forms, fitted to the MXFP4 blocks of
32 that gfx950's FP4 matrix instruction scales):

  * Random Hadamard transform (RHT): along the Wgrad reduction axis (tokens), in blocks
    of 16 consecutive rows, y = (1/4) H16 diag(s) x with H16 the Sylvester Hadamard
    matrix and s a random sign vector (a 16-bit mask, bit j set -> s_j = -1) drawn by
    the caller per step and shared by both Wgrad operands.  Q = H16 diag(s) / 4 is
    orthogonal, so dY'^T X' = dY^T Q^T Q X = dY^T X: the transform changes the
    quantization error, not the product.  The sum is formed by the fast transform's
    butterflies (pairs i, i + h for h = 1, 2, 4, 8: a + b, a - b) in float64, which is
    exact while the 16 inputs' exponents span less than about 41 bits (always on the
    synthetic data), then scaled by 1/4 (exact) and rounded once to fp32.  The column
    copy of the MXFP4 quantization is then taken of y.
  * Stochastic rounding (SR) of the E2M1 elements of gradient copies: for a scaled
    magnitude a < 6 between neighbouring E2M1 magnitudes lo <= a < hi, round up iff
    r < p 2^16 with p = (a - lo) / (hi - lo) (exact in fp32: hi - lo is a power of two
    and a - lo exact), r a 16-bit uniform integer; a >= 6 saturates to 6; the sign is
    kept.  The block scale is the MXFP4 rule (unchanged).  The random integers come
    from the counter-based generator Philox4x64-10 (Salmon et al., SC'11): element
    (r, c) of a copy with C columns has index i = r C + c; call i // 16 with counter
    (i // 16, copy, 0, 0) and key (seed, 0); r = 16-bit lane i % 16 of the four 64-bit
    outputs (lane l: word l // 4, bits 16 (l % 4) ..).  copy = 0 for the row-wise copy,
    1 for the column-wise copy.
  * 2D block scaling of weights: one E8M0 scale per 32 x 32 tile (the MXFP4 rule on the
    tile's amax); the row-wise copy repeats the tile's scale for each of its 32 rows'
    blocks and the column-wise copy is its transpose (same codes), so W and W^T are one
    quantization.
  * The extra per-tensor amax pass belongs to NVFP4's second-level fp32 scale; MXFP4's
    E8M0 block scales need no per-tensor scale, so there is no such pass here.

Pins (tests/test_oracle_fp4_recipe.py): H16 against scipy.linalg.hadamard and
H H^T = 16 I; the transform against the matrix product on integer data, its exact
inverse, and the Wgrad product preserved; Philox4x64-10 against numpy.random.Philox's
raw output; SR exhaustively over all 2^16 random values (the up-rounding count and the
mean), on-grid values unchanged; 2D codes in closed form, the transpose property and
the reduction to the 1D quantizer.
"""

from __future__ import annotations

import numpy as np

from .mxfp4 import BLOCK, _MAGS, block_exponent, e2m1_encode, pack

MASK64 = (1 << 64) - 1
# Philox4x64 multipliers and key increments (Salmon, Moraes, Dror, Shaw, "Parallel random
# numbers: as easy as 1, 2, 3", SC'11)
PHILOX_M0, PHILOX_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
PHILOX_W0, PHILOX_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def hadamard(n: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order n (a power of two), float64."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _signs(sign_mask: int) -> np.ndarray:
    return np.array([-1.0 if (sign_mask >> j) & 1 else 1.0 for j in range(16)])


def rht16_rows(x, sign_mask: int) -> np.ndarray:
    """The random Hadamard transform of the reading above along axis 0 (rows) of x [R, C]
    (R % 16 == 0): fp32 result."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    R, C = x64.shape
    if R % 16:
        raise ValueError("rows must be a multiple of 16")
    v = x64.reshape(R // 16, 16, C) * _signs(sign_mask)[None, :, None]
    h = 1
    while h < 16:  # butterflies: within blocks of 2h, (a, b) -> (a + b, a - b)
        v = v.reshape(R // 16, 16 // (2 * h), 2, h, C)
        a, b = v[:, :, 0].copy(), v[:, :, 1].copy()
        v = np.stack([a + b, a - b], axis=2).reshape(R // 16, 16, C)
        h *= 2
    return (v * 0.25).reshape(R, C).astype(np.float32)


def _mulhilo64(a: int, b: np.ndarray):
    """(hi, lo) 64-bit halves of a * b for a constant a and uint64 array b (exact)."""
    b = b.astype(np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    a0, a1 = np.uint64(a & 0xFFFFFFFF), np.uint64(a >> 32)
    b0, b1 = b & m32, b >> np.uint64(32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> np.uint64(32)) + (p01 & m32) + (p10 & m32)
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    lo = (p00 & m32) | ((mid & m32) << np.uint64(32))
    return hi, lo


def philox4x64_10(counters, key) -> np.ndarray:
    """Philox4x64 with 10 rounds: counters [n, 4] uint64, key (k0, k1) -> [n, 4] uint64."""
    c = np.array(counters, dtype=np.uint64).reshape(-1, 4)
    c0, c1, c2, c3 = (c[:, i].copy() for i in range(4))
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0, k1 = (k0 + PHILOX_W0) & MASK64, (k1 + PHILOX_W1) & MASK64
            hi0, lo0 = _mulhilo64(PHILOX_M0, c0)
            hi1, lo1 = _mulhilo64(PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=1)


def sr_bits16(rows: int, cols: int, copy: int, seed: int, first_row: int = 0) -> np.ndarray:
    """The 16-bit random integers of the elements (r, c) of rows first_row .. first_row +
    rows - 1 of a copy with `cols` columns (element index i = r cols + c)."""
    i0 = first_row * cols
    n = rows * cols
    c_lo, c_hi = i0 // 16, -(-(i0 + n) // 16)
    ctr = np.zeros((c_hi - c_lo, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(c_lo, c_hi, dtype=np.uint64)
    ctr[:, 1] = np.uint64(copy)
    out = philox4x64_10(ctr, (seed, 0))                       # [calls, 4] uint64
    lanes = np.empty((c_hi - c_lo, 16), dtype=np.uint16)
    for l in range(16):
        lanes[:, l] = ((out[:, l // 4] >> np.uint64(16 * (l % 4))) & np.uint64(0xFFFF)).astype(np.uint16)
    start = i0 - 16 * c_lo
    return lanes.reshape(-1)[start:start + n].reshape(rows, cols)


def e2m1_encode_sr(y, r16) -> np.ndarray:
    """Stochastic rounding of scaled values y to E2M1 codes with the 16-bit integers r16."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    idx = np.searchsorted(_MAGS, np.minimum(a, 6.0), side="right") - 1   # lo = _MAGS[idx] <= a
    idx = np.minimum(idx, 7)
    lo = _MAGS[idx]
    hi = _MAGS[np.minimum(idx + 1, 7)]
    width = np.where(idx < 7, hi - lo, 1.0)
    p = (a - lo) / width
    up = (idx < 7) & (np.asarray(r16, dtype=np.float64) < p * 65536.0)
    code = np.where(a >= 6.0, 7, idx + up)
    sign = np.where(np.signbit(y) & ~nan, 8, 0)
    return (code + sign).astype(np.uint8)


def mxfp4_quantize_sr(x, seed: int, copy: int, first_row: int = 0):
    """MXFP4 of the rows of x with stochastic rounding of the elements: (packed [R, C/2],
    e8m0 [R, C/32]); the rows of x are rows first_row .. of the copy, and the random
    integers of element (r, c) are those of sr_bits16."""
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    xb = x32.reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    e, codes = block_exponent(xb)
    scaled = np.ldexp(xb, (-e)[:, :, None].astype(np.int32)).astype(np.float32)
    q = e2m1_encode_sr(scaled.reshape(R, C), sr_bits16(R, C, copy, seed, first_row))
    return pack(q), codes


def mxfp4_quantize_2d(w):
    """2D block-scaled MXFP4 of w [R, C] (both multiples of 32): returns (row packed
    [R, C/2], row e8m0 [R, C/32], column packed [C, R/2], column e8m0 [C, R/32])."""
    w32 = np.asarray(w, dtype=np.float32)
    R, C = w32.shape
    if R % BLOCK or C % BLOCK:
        raise ValueError("2D blocks need rows and cols that are multiples of 32")
    t = w32.reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK).transpose(0, 2, 1, 3).astype(np.float64)
    tiles = t.reshape(R // BLOCK, C // BLOCK, BLOCK * BLOCK)
    e, tcodes = block_exponent(tiles)                     # [R/32, C/32]
    scaled = np.ldexp(t, (-e)[:, :, None, None].astype(np.int32))
    codes = e2m1_encode(scaled.transpose(0, 2, 1, 3).reshape(R, C))
    row_scale = np.repeat(tcodes, BLOCK, axis=0)          # [R, C/32]
    col_scale = np.repeat(tcodes.T, BLOCK, axis=0)        # [C, R/32]
    return pack(codes), row_scale, pack(np.ascontiguousarray(codes.T)), col_scale
