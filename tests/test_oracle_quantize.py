"""Pins for the oracle's amax, scale, scaled cast, delayed history and MXFP8 quantizer.

Each test checks the oracle against something other than itself: a Python
loop, a closed form fixed by the scale relation scale = fp8_max / amax, an
invariant of current scaling, the delayed-history closed forms (constant input,
a spike, most_recent, a drifting input), or the per-element encoder (pinned in
test_oracle_formats.py).
"""

import json
import os

import numpy as np
import pytest

import oracle as O

from oracle import (E4M3, E5M2, DelayedScalingState, amax, current_scale, decode_table,
                    delayed_update, encode, mxfp8_quantize, scale_inverse, scaled_cast,
                    cast_transpose)

FLT_MAX = np.float32(np.finfo(np.float32).max)
GOLD = os.path.join(os.path.dirname(__file__), "golden", "recipe_constants.json")


def test_amax_python_loop_and_planted_max():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 53)).astype(np.float32)
    m = 0.0
    for v in x.reshape(-1):
        m = max(m, abs(float(v)))
    assert amax(x) == np.float32(m)
    x[5, 7] = -123.5
    assert amax(x) == np.float32(123.5)
    perm = rng.permutation(x.size)
    assert amax(x.reshape(-1)[perm]) == amax(x)
    assert amax(np.array([-0.0, 0.0], dtype=np.float32)) == 0.0
    assert amax(np.zeros((0, 4), dtype=np.float32)) == 0.0


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_current_scale_closed_forms(fmt):
    mx = np.float32(fmt.max)
    assert current_scale(mx, fmt) == 1.0
    for k in range(-20, 20):
        # power-of-two amax: the division is exact
        assert current_scale(np.float32(2.0 ** k), fmt) == np.float32(fmt.max * 2.0 ** -k)
    assert current_scale(0.0, fmt) == 1.0
    assert current_scale(np.inf, fmt) == 1.0
    assert current_scale(np.nan, fmt) == 1.0
    assert current_scale(np.finfo(np.float32).smallest_subnormal, fmt) == FLT_MAX
    assert current_scale(np.float32(fmt.max), fmt, margin=2) == 0.25
    assert scale_inverse(np.float32(4.0)) == 0.25
    # margin halves the scale per unit
    assert current_scale(np.float32(3.0), fmt, margin=1) == np.float32(np.float32(fmt.max / 3.0) / 2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
@pytest.mark.parametrize("seed", range(6))
def test_current_scaling_amax_element_hits_max_code(fmt, seed):
    """Invariant: with scale = fp8_max/amax, the amax element encodes to +-max exactly,
    and every other code stays within [-max, max]."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, (64, 96)) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
    a = amax(x)
    s = current_scale(a, fmt)
    q = scaled_cast(x, s, fmt)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert (q[i] & 0x7F) == fmt.max_code
    v = decode_table(fmt)[q]
    assert np.all(np.abs(v) <= fmt.max)


def test_scaled_cast_reduces_to_encode():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096).astype(np.float32) * 30
    np.testing.assert_array_equal(scaled_cast(x, 1.0, E4M3), encode(x, E4M3))
    # a power-of-two scale is exact in fp32, so the cast equals the encode of the exact product
    np.testing.assert_array_equal(scaled_cast(x, 0.125, E5M2), encode(x / 8, E5M2))


def test_cast_transpose_is_byte_transpose():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((48, 80)).astype(np.float32)
    row, col = cast_transpose(x, np.float32(3.5), E4M3)
    np.testing.assert_array_equal(row, scaled_cast(x, np.float32(3.5), E4M3))
    assert col.shape == (80, 48)
    for r in range(48):
        for c in range(80):
            assert col[c, r] == row[r, c]


def test_recipe_constants_from_pages():
    with open(GOLD) as f:
        g = json.load(f)
    st = DelayedScalingState(E4M3, g["example_amax_history_len"], g["example_amax_compute_algo"],
                             g["nemo_fp8_margin"])
    assert st.hist.shape == (16,) and st.scale == 1.0 and st.scale_inv == 1.0


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_delayed_constant_input(fmt):
    """Constant input c: scale_0 = 1 (initial), scale_t = fp8_max / c for t >= 1."""
    c = np.float32(0.37)
    st = DelayedScalingState(fmt, 16, "max")
    scales = []
    for t in range(20):
        scales.append(st.scale)
        st.cast(np.full((4, 8), c, dtype=np.float32))
        st.update()
    assert scales[0] == 1.0
    for t in range(1, 20):
        assert scales[t] == np.float32(np.float32(fmt.max) / c)


def test_delayed_spike_dominates_exactly_sixteen_steps():
    base, spike, k = np.float32(1.0), np.float32(64.0), 3
    st = DelayedScalingState(E4M3, 16, "max")
    used = []
    for t in range(40):
        used.append(st.scale)
        v = spike if t == k else base
        st.cast(np.full((2, 2), v, dtype=np.float32))
        st.update()
    for t in range(1, 40):
        expect = np.float32(448.0) / (spike if k + 1 <= t <= k + 16 else base)
        assert used[t] == np.float32(expect), t


def test_delayed_most_recent():
    rng = np.random.default_rng(4)
    st = DelayedScalingState(E5M2, 16, "most_recent")
    prev = None
    for t in range(12):
        x = rng.standard_normal((8, 8)).astype(np.float32) * np.float32(2.0 ** rng.integers(-5, 5))
        if prev is not None:
            assert st.scale == np.float32(np.float32(57344.0) / prev)
        st.cast(x)
        st.update()
        prev = np.float32(np.max(np.abs(x)))


def test_delayed_keeps_scale_on_zero_history_and_rolls():
    h = np.zeros(4, dtype=np.float32)
    nh, s, si = delayed_update(h, np.float32(8.0), E4M3)
    assert s == 8.0 and si == 0.125 and (nh == 0).all()
    h = np.array([3.0, 5.0, 1.0, 2.0], dtype=np.float32)
    nh, s, si = delayed_update(h, np.float32(1.0), E4M3)
    np.testing.assert_array_equal(nh, [0.0, 3.0, 5.0, 1.0])
    assert s == np.float32(448.0 / 5.0)
    nh, s, _ = delayed_update(np.array([np.inf, 1, 1, 1], dtype=np.float32), np.float32(2.0), E4M3)
    assert s == 2.0
    nh, s, _ = delayed_update(np.array([1e-45, 0, 0, 0], dtype=np.float32), np.float32(2.0), E4M3)
    assert s == FLT_MAX


def test_delayed_drift_saturation_count():
    """Input growing x1.05 per step: the scale for step t+1 is fp8_max/amax_t, so the
    elements of x_{t+1} above amax_t saturate -- a count fixed by the data alone."""
    rng = np.random.default_rng(5)
    base = rng.standard_normal((64, 64)).astype(np.float32)
    st = DelayedScalingState(E4M3, 16, "most_recent")
    prev_amax = None
    for t in range(6):
        x = (base * np.float32(1.05 ** t)).astype(np.float32)
        q, _ = st.cast(x)
        if prev_amax is not None:
            prod = np.abs(x * st.scale)
            # the elements that grew past amax_t (by the factor 1.05) saturate
            n_over = int(np.sum(np.abs(x) > prev_amax))
            assert n_over >= 1
            assert int(np.sum(prod > np.float32(448.0))) == n_over
            # max code = saturated values plus those rounding to 448 from above the
            # 416/448 midpoint (432, a tie that goes to the even mantissa of 448)
            n_max = int(np.sum((q & 0x7F) == E4M3.max_code))
            assert n_max == int(np.sum(prod >= np.float32(432.0)))
        st.update()
        prev_amax = np.max(np.abs(x))


def test_mxfp8_closed_form_codes():
    rng = np.random.default_rng(6)
    R, C = 8, 128
    x = rng.standard_normal((R, C)).astype(np.float32)
    # plant a known block amax per block: 2^j * 1.5 -> floor(log2) = j -> code j - 8 + 127
    js = rng.integers(-30, 30, (R, C // 32))
    for r in range(R):
        for b in range(C // 32):
            blk = x[r, b * 32:(b + 1) * 32]
            blk[:] = np.clip(blk, -1.0, 1.0) * np.float32(2.0 ** int(js[r, b]))
            blk[int(rng.integers(0, 32))] = np.float32(1.5 * 2.0 ** int(js[r, b]))
    q, e = mxfp8_quantize(x)
    np.testing.assert_array_equal(e.astype(int), js - 8 + 127)
    # elements are the per-element encode of x * 2^-(code-127)
    for r in range(R):
        for b in range(C // 32):
            sc = np.float32(2.0 ** -(int(e[r, b]) - 127))
            np.testing.assert_array_equal(q[r, b * 32:(b + 1) * 32],
                                          encode(x[r, b * 32:(b + 1) * 32] * sc, E4M3))


def test_mxfp8_zero_block_and_clamp():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = np.float32(2.0 ** 120)
    q, e = mxfp8_quantize(x)
    assert e[0, 0] == 127 and e[0, 1] == 127 and e[1, 0] == 127
    assert e[1, 1] == 120 - 8 + 127
    # 2^120 / 2^112 = 2^8 = 256: E4M3 exponent field 8 + 7 = 15, mantissa 0 -> 0x78
    assert (q[1, 32:] == 0x78).all()
    # the shared exponent clamps at -127 (code 0) for a block of fp32 subnormals
    y = np.full((1, 32), np.finfo(np.float32).smallest_subnormal, dtype=np.float32)
    qy, ey = mxfp8_quantize(y)
    assert ey[0, 0] == 0 and (qy == 0).all()


def test_mxfp8_e5m2_closed_form_codes():
    """E5M2 elements (largest power of two 2^15): block code floor(log2 amax) - 15 + 127,
    worked by hand for a block of max 1.5 * 2^j: the max scales to 1.5 * 2^15 = 49152,
    E5M2 exponent field 30, mantissa 10 -> 0x7A; 1.9 * 2^j scales into [57344, 65536) and
    saturates to 0x7B; 2^(j-30), 2^(j-31), 2^(j-32) scale to 2^-15, 2^-16 (two and one
    times the smallest subnormal: codes 0x02, 0x01) and 2^-17 (the tie between 0 and
    2^-16, to even: 0x00)."""
    for j in (-20, 0, 7, 40):
        x = np.zeros((2, 32), dtype=np.float32)
        x[0, 0] = np.float32(1.5 * 2.0 ** j)
        x[0, 1] = np.float32(-(2.0 ** (j - 30)))
        x[0, 2] = np.float32(2.0 ** (j - 31))
        x[0, 3] = np.float32(2.0 ** (j - 32))
        x[1, 5] = np.float32(-1.9 * 2.0 ** j)
        x[1, 6] = np.float32(1.0 * 2.0 ** j)
        q, e = mxfp8_quantize(x, E5M2)
        assert e[0, 0] == j - 15 + 127 and e[1, 0] == j - 15 + 127
        assert q[0, 0] == 0x7A and q[0, 1] == 0x82 and q[0, 2] == 0x01 and q[0, 3] == 0x00
        assert q[1, 5] == 0xFB                 # -1.9 * 2^15 saturates to -57344
        assert q[1, 6] == 0x78                 # 2^15: exponent field 30, mantissa 0
        assert (q[0, 4:] == 0).all() and q[1, 0] == 0


def test_mxfp8_e5m2_zero_block_and_clamp():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = np.float32(2.0 ** 120)
    q, e = mxfp8_quantize(x, E5M2)
    assert e[0, 0] == 127 and e[0, 1] == 127 and e[1, 0] == 127   # all-zero blocks
    assert e[1, 1] == 120 - 15 + 127
    assert (q[1, 32:] == 0x78).all()   # 2^120 / 2^105 = 2^15
    assert (q[0] == 0).all()
    # fp32 subnormals: floor(log2) = -149, e = -164 clamps to -127 (code 0); the
    # elements scale to 2^-22, below E5M2's smallest subnormal 2^-16: +0
    y = np.full((1, 32), np.finfo(np.float32).smallest_subnormal, dtype=np.float32)
    qy, ey = mxfp8_quantize(y, E5M2)
    assert ey[0, 0] == 0 and (qy == 0).all()
    # e = -127 exactly (amax 2^-112) keeps the scaled elements in range: 2^-112 * 2^127 = 2^15
    z = np.zeros((1, 32), dtype=np.float32)
    z[0, 0] = np.float32(2.0 ** -112)
    qz, ez = mxfp8_quantize(z, E5M2)
    assert ez[0, 0] == 0 and qz[0, 0] == 0x78


def test_mxfp8_infinite_and_nan_blocks():
    """An infinite block max has log2 = +inf, so the exponent takes the clamp's top, 127
    (code 254): the infinities saturate to the format's largest magnitude and finite
    elements, divided by 2^127, round to zero. A NaN makes the block max NaN, which is
    not > 0, so that block keeps e = 0 (code 127) and its NaN stays a NaN."""
    x = np.zeros((1, 96), dtype=np.float32)
    x[0, 0], x[0, 1], x[0, 2] = np.inf, 3.0, -np.float32(2.0 ** 100)
    x[0, 32], x[0, 33], x[0, 34] = -np.inf, np.nan, 1.5
    x[0, 64], x[0, 65] = np.inf, -np.inf
    for fmt, top in ((E4M3, 0x7E), (E5M2, 0x7B)):
        q, e = mxfp8_quantize(x, fmt)
        assert list(e[0]) == [254, 127, 254]
        assert q[0, 0] == top and q[0, 1] == 0 and q[0, 2] == 0x80  # -2^100 / 2^127 -> -0
        assert q[0, 32] == top | 0x80 and np.isnan(O.decode_table(fmt)[q[0, 33]])
        assert q[0, 34] == encode(np.float32(1.5), fmt)           # scale 2^0
        assert q[0, 64] == top and q[0, 65] == top | 0x80


def test_mx_scales_panel_layout_positions():
    """The panel layout of the MX scales, pinned at positions worked out by hand from
    its definition: 256-row panels; in a panel, the dwords (four block bytes) of one
    128-element group for all 256 rows are contiguous."""
    R, nb = 3, 8  # 256 columns: two groups of four blocks
    e = np.array([[10 * r + b for b in range(nb)] for r in range(R)], np.uint8)
    p = O.mx_scales_panel(e)
    assert p.shape == (256 * 2 * 4,)
    assert p[0] == 0 and p[3] == 3          # row 0, blocks 0 and 3: first dword of group 0
    assert p[4] == 10                       # row 1, block 0: the next dword
    assert p[1024] == 4                     # row 0, block 4: group 1 starts after 256 dwords
    assert p[1024 + 8 + 1] == 25            # row 2, block 5
    assert p[1024 + 8 + 3] == 27            # row 2, block 7
    assert p[12] == 127 and p[1024 + 1020] == 127  # padding rows 3 and 255
    # second panel: 300 rows, 384 columns (three groups); row 257 block 2
    e2 = np.zeros((300, 12), np.uint8)
    e2[257, 2] = 200
    p2 = O.mx_scales_panel(e2)
    assert p2.shape == (2 * 256 * 3 * 4,)
    assert p2[4 * (1 * 3 + 0) * 256 + 4 * 1 + 2] == 200
    assert int(np.count_nonzero(p2 == 200)) == 1


def test_mx_scales_panel_round_trip():
    rng = np.random.default_rng(11)
    for R, nb in ((1, 4), (255, 8), (256, 4), (300, 12), (513, 16)):
        e = rng.integers(0, 256, (R, nb)).astype(np.uint8)
        np.testing.assert_array_equal(O.mx_scales_from_panel(O.mx_scales_panel(e), R, nb), e)
    with pytest.raises(ValueError):
        O.mx_scales_panel(np.zeros((4, 6), np.uint8))
