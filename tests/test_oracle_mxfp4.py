"""Pins of the MXFP4 oracle (CPU only)."""

import numpy as np

from oracle import mxfp4 as F
from oracle.quantize import e8m0_to_float


def test_table_from_bit_fields():
    t = F.e2m1_decode_table()
    np.testing.assert_array_equal(t[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(t[8:], -t[:8])
    assert np.signbit(t[8])


def test_round_trip_every_code():
    t = F.e2m1_decode_table()
    np.testing.assert_array_equal(F.e2m1_encode(t), np.arange(16))


def test_midpoint_ties_go_to_the_even_mantissa():
    # (lower neighbour, upper neighbour, the one with the even mantissa)
    cases = [(0.0, 0.5, 0.0), (0.5, 1.0, 1.0), (1.0, 1.5, 1.0), (1.5, 2.0, 2.0), (2.0, 3.0, 2.0),
             (3.0, 4.0, 4.0), (4.0, 6.0, 4.0)]
    t = F.e2m1_decode_table()
    for lo, hi, even in cases:
        mid = (lo + hi) / 2
        assert t[F.e2m1_encode(mid)] == even, mid
        assert t[F.e2m1_encode(-mid)] == -even, -mid
        assert t[F.e2m1_encode(np.nextafter(mid, 10.0))] == hi, mid
        assert t[F.e2m1_encode(np.nextafter(mid, -10.0))] == lo, mid


def test_saturation_and_monotone():
    t = F.e2m1_decode_table()
    assert t[F.e2m1_encode(6.5)] == 6 and t[F.e2m1_encode(1e30)] == 6 and t[F.e2m1_encode(-np.inf)] == -6
    x = np.linspace(-8, 8, 20001)
    v = t[F.e2m1_encode(x)]
    assert np.all(np.diff(v) >= 0)
    assert np.all(np.abs(v - np.clip(x, -6, 6)) <= 1.0 + 1e-12)


def test_block_scales_closed_form():
    x = np.zeros((3, 64), np.float32)
    x[0, :32] = 6.0 * 2.0 ** 5          # amax 6 * 2^5 -> e = 5, code 132, elements exactly +-6
    x[0, 32:] = 0.0                    # all zero -> code 127
    x[1, 5] = 1.0                      # amax 1 = 2^0 -> e = -2
    x[1, 40] = -3.0 * 2.0 ** -130      # tiny -> clamped to -127
    x[2, 7] = np.nan
    x[2, 40] = -np.inf                 # infinite amax -> e = 127 (code 254)
    x[2, 41] = 1.0e30                  # finite, 1e30 * 2^-127 < 0.25 -> 0
    q, e = F.mxfp4_quantize(x)
    np.testing.assert_array_equal(e[0], [132, 127])
    assert e[1, 0] == 125 and e[1, 1] == 0 and e[2, 0] == 255 and e[2, 1] == 254
    codes = F.unpack(q)
    assert np.all(F.e2m1_decode_table()[codes[0, :32]] == 6.0)
    assert F.e2m1_decode_table()[codes[1, 5]] == 4.0   # 1 * 2^2
    assert codes[2, 7] == 0
    assert codes[2, 40] == 15 and codes[2, 41] == 0   # -6 and +0


def test_pack_layout():
    c = np.arange(16, dtype=np.uint8).reshape(1, 16)
    p = F.pack(c)
    np.testing.assert_array_equal(p[0], [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE])
    np.testing.assert_array_equal(F.unpack(p), c)


def test_gemm_brute_force_and_unit_scales():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((5, 64)).astype(np.float32) * 4
    b = rng.standard_normal((3, 64)).astype(np.float32) / 3
    qa, ea = F.mxfp4_quantize(a)
    qb, eb = F.mxfp4_quantize(b)
    t = F.e2m1_decode_table()
    ca, cb = F.unpack(qa), F.unpack(qb)
    d = F.gemm_mxfp4(qa, ea, qb, eb, out="f32")
    for i in range(5):
        for j in range(3):
            s = sum(t[ca[i, k]] * e8m0_to_float(ea[i, k // 32]) * t[cb[j, k]] * e8m0_to_float(eb[j, k // 32])
                    for k in range(64))
            assert d[i, j] == np.float32(s)
    one_a = np.full(ea.shape, 127, np.uint8)
    one_b = np.full(eb.shape, 127, np.uint8)
    np.testing.assert_array_equal(F.gemm_mxfp4(qa, one_a, qb, one_b, out="f32"),
                                  (t[ca] @ t[cb].T).astype(np.float32))
