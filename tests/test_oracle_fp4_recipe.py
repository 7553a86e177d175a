"""Pins of oracle/fp4_recipe.py: the random Hadamard transform, Philox4x64-10 and the
stochastic rounding it drives, and the 2D block scaling of weights.  Each checks the
oracle against something other than itself: a library routine (scipy's Hadamard
matrix, numpy's Philox generator), exact rational arithmetic, exhaustive enumeration of
the random integers, closed forms, or the 1D quantizer pinned elsewhere."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O
from oracle.mxfp4 import dequantize, e2m1_decode_table, mxfp4_quantize, unpack


def test_hadamard_is_sylvester_and_orthogonal():
    H = O.hadamard(16)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(16))
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16))


@pytest.mark.parametrize("mask", [0x0000, 0xFFFF, 0x8001, 0x5A3C])
def test_rht_matches_the_matrix_product_on_integers(mask):
    rng = np.random.default_rng(mask)
    x = rng.integers(-100, 101, (64, 5)).astype(np.float32)
    y = O.rht16_rows(x, mask)
    s = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
    H = scipy.linalg.hadamard(16).astype(np.float64)
    for b in range(4):
        blk = x[16 * b:16 * b + 16].astype(np.float64)
        np.testing.assert_array_equal(y[16 * b:16 * b + 16], ((H @ (s[:, None] * blk)) / 4).astype(np.float32))
        # exact inverse: x = diag(s) H y / 4
        np.testing.assert_array_equal(s[:, None] * (H @ y[16 * b:16 * b + 16].astype(np.float64)) / 4, blk)


def test_rht_preserves_the_wgrad_product():
    """The same signs on both Wgrad operands: dY'^T X' = dY^T X exactly (integer data)."""
    rng = np.random.default_rng(3)
    dy = rng.integers(-20, 21, (48, 6)).astype(np.float32)
    x = rng.integers(-20, 21, (48, 7)).astype(np.float32)
    mask = 0x2B71
    lhs = O.rht16_rows(dy, mask).astype(np.float64).T @ O.rht16_rows(x, mask).astype(np.float64)
    np.testing.assert_array_equal(lhs, dy.astype(np.float64).T @ x.astype(np.float64))


def test_rht_is_the_exact_sum_rounded_once():
    """On bf16 activations the float64 butterflies are exact: the result equals the
    exact rational transform rounded once to fp32."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 3)).astype(np.float32)
    x[::7] *= 50
    x = O.bf16_bits_to_f32(O.bf16_round_bits(x))
    mask = 0xC0DE
    y = O.rht16_rows(x, mask)
    H = scipy.linalg.hadamard(16)
    s = [-1 if (mask >> j) & 1 else 1 for j in range(16)]
    for b in range(2):
        for c in range(3):
            for i in range(16):
                exact = sum(Fraction(int(H[i, j]) * s[j]) * Fraction(float(x[16 * b + j, c])) for j in range(16)) / 4
                assert y[16 * b + i, c] == np.float32(float(exact))


@pytest.mark.parametrize("ctr,key", [(1, 0), (6, 7), (123456790 + (3 << 64) + (9 << 128), (11 << 64) + 42),
                                     ((1 << 64) + 1, 5), (2 ** 200 + 77, (1 << 127) + 3)])
def test_philox_matches_numpy(ctr, key):
    """numpy's Philox (4x64, 10 rounds) advances its counter by one before each block of
    four outputs, so its output from counter c - 1 is Philox of counter c."""
    g = np.random.Philox(counter=ctr - 1, key=key)
    ref = np.array([int(v) for v in g.random_raw(4)], dtype=np.uint64)
    words = [(ctr >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    got = O.philox4x64_10([words], (key & ((1 << 64) - 1), key >> 64))[0]
    np.testing.assert_array_equal(got, ref)


def test_philox_stream_of_counters_matches_numpy():
    g = np.random.Philox(counter=0, key=(9 << 64) + 1234)
    ref = np.array([int(v) for v in g.random_raw(4 * 100)], dtype=np.uint64).reshape(100, 4)
    ctr = np.zeros((100, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(1, 101, dtype=np.uint64)
    np.testing.assert_array_equal(O.philox4x64_10(ctr, (1234, 9)), ref)


def test_sr_bits_follow_the_linear_index_and_differ_by_copy_and_seed():
    a = O.sr_bits16(4, 48, 0, 99)
    np.testing.assert_array_equal(a.reshape(-1), O.sr_bits16(1, 192, 0, 99).reshape(-1))
    np.testing.assert_array_equal(a.reshape(-1)[:96], O.sr_bits16(6, 16, 0, 99).reshape(-1))
    np.testing.assert_array_equal(O.sr_bits16(2, 48, 0, 99, first_row=1), a[1:3])   # rows of a copy
    np.testing.assert_array_equal(O.sr_bits16(3, 40, 1, 5, first_row=2), O.sr_bits16(6, 40, 1, 5)[2:5])
    assert not np.array_equal(a, O.sr_bits16(4, 48, 1, 99))
    assert not np.array_equal(a, O.sr_bits16(4, 48, 0, 98))
    big = O.sr_bits16(256, 256, 0, 7).astype(np.int64)
    counts = np.bincount(big.reshape(-1) >> 12, minlength=16)  # 16 equal bins of the 16-bit range
    chi2 = float(((counts - 4096) ** 2 / 4096).sum())
    assert chi2 < 50.0  # 15 degrees of freedom: p < 1e-5 beyond this


@pytest.mark.parametrize("v,lo,hi", [(0.3, 0.0, 0.5), (1.25, 1.0, 1.5), (2.75, 2.0, 3.0), (5.0, 4.0, 6.0),
                                     (1e-4, 0.0, 0.5), (5.999, 4.0, 6.0), (0.5, 0.5, 1.0)])
def test_sr_exhaustive_over_the_random_integers(v, lo, hi):
    """Over all 2^16 random integers: round up exactly ceil(p 2^16) times (p 2^16 times
    when it is an integer), so the mean is within (hi - lo) 2^-16 of v; negative values
    are the mirror image."""
    r = np.arange(65536, dtype=np.uint16)
    vv = np.float32(v)
    codes = O.e2m1_encode_sr(np.full(65536, vv, np.float32), r)
    vals = e2m1_decode_table()[codes]
    assert set(np.unique(vals)) <= {lo, hi}
    p = (float(vv) - lo) / (hi - lo)
    n_up = int(np.sum(vals == hi)) if hi != lo else 0
    expect = int(np.ceil(p * 65536.0)) if p * 65536.0 != int(p * 65536.0) else int(p * 65536.0)
    assert n_up == expect
    assert abs(vals.mean() - float(vv)) <= (hi - lo) * 2.0 ** -16
    neg = O.e2m1_encode_sr(np.full(65536, -vv, np.float32), r)
    np.testing.assert_array_equal(neg, codes | 8)


def test_sr_grid_values_saturation_and_nan():
    r = np.arange(0, 65536, 97, dtype=np.uint16)
    for g in (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0):
        c = O.e2m1_encode_sr(np.full(r.size, g, np.float32), r)
        assert (e2m1_decode_table()[c] == g).all()
    for big in (6.0, 7.9, 1e30, np.inf):
        assert (O.e2m1_encode_sr(np.full(r.size, big, np.float32), r) == 7).all()
    assert (O.e2m1_encode_sr(np.full(r.size, np.nan, np.float32), r) == 0).all()
    assert (O.e2m1_encode_sr(np.full(r.size, -0.0, np.float32), r) == 8).all()


def test_mxfp4_sr_keeps_the_block_scales_and_is_unbiased():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, (64, 256)) * 1e-3).astype(np.float32)
    q_rne, e_rne = mxfp4_quantize(x)
    q_sr, e_sr = O.mxfp4_quantize_sr(x, seed=17, copy=0)
    np.testing.assert_array_equal(e_sr, e_rne)
    v = dequantize(q_sr, e_sr)
    scale = np.repeat(O.e8m0_to_float(e_sr), 32, axis=1)
    # each element one of the two grid neighbours of its scaled value
    y = x / scale
    lo = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.abs(y)
    idx = np.clip(np.searchsorted(lo, a, side="right") - 1, 0, 7)
    ok = (np.abs(v / scale) == lo[idx]) | (np.abs(v / scale) == lo[np.minimum(idx + 1, 7)])
    assert ok.all()
    # unbiased: the mean error over 16384 elements is far below one grid step
    err = (v - x) / scale
    assert abs(err.mean()) < 0.01 and abs(err).max() <= 2.0
    assert not np.array_equal(q_sr, q_rne)


def test_2d_block_codes_closed_form_and_transpose():
    rng = np.random.default_rng(6)
    R, C = 64, 96
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    js = rng.integers(-12, 0, (R // 32, C // 32))
    for i in range(R // 32):
        for j in range(C // 32):
            t = w[32 * i:32 * i + 32, 32 * j:32 * j + 32]
            t[:] = np.clip(t, -2.0 ** int(js[i, j]), 2.0 ** int(js[i, j]))
            t[int(rng.integers(0, 32)), int(rng.integers(0, 32))] = np.float32(1.5 * 2.0 ** int(js[i, j]))
    qr, er, qc, ec = O.mxfp4_quantize_2d(w)
    np.testing.assert_array_equal(er[::32], js - 2 + 127)           # floor(log2 1.5 2^j) - 2 + 127
    np.testing.assert_array_equal(er, np.repeat(js - 2 + 127, 32, axis=0))
    np.testing.assert_array_equal(ec, np.repeat((js - 2 + 127).T, 32, axis=0))
    np.testing.assert_array_equal(unpack(qc), unpack(qr).T)          # W^T is the same quantization
    np.testing.assert_array_equal(dequantize(qc, ec), dequantize(qr, er).T)


def test_2d_reduces_to_1d_when_every_row_holds_the_tile_max():
    rng = np.random.default_rng(7)
    R, C = 64, 64
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    for i in range(R // 32):
        for j in range(C // 32):
            t = w[32 * i:32 * i + 32, 32 * j:32 * j + 32]
            m = np.float32(np.abs(t).max() * 1.01)
            t[np.arange(32), rng.integers(0, 32, 32)] = m  # every row of the tile reaches the tile max
    qr, er, _, _ = O.mxfp4_quantize_2d(w)
    q1, e1 = mxfp4_quantize(w)
    np.testing.assert_array_equal(qr, q1)
    np.testing.assert_array_equal(er, e1)
