"""Pins for the oracle's GEMMs (per-tensor FP8, MXFP8, BF16) and its bf16 rounding.

Checks against: a Python triple loop with exact rational sums, integer-valued
operands compared with an int64 matmul, the identity operand, bias-only
(A = 0), power-of-two scale linearity, MX with all scale codes 127 equal to
per-tensor, MX block decomposition on 1x1 outputs by brute force, and
PyTorch's CPU fp32 -> bf16 conversion.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

from oracle import (E4M3, E5M2, bias_grad, bf16_bits_to_f32, bf16_round_bits, decode, decode_table,
                    encode, gemm_bf16, gemm_mx, gemm_per_tensor, rel_err, e8m0_to_float)


def _rand_codes(rng, shape, fmt):
    """Random finite codes (no NaN/Inf)."""
    t = decode_table(fmt)
    ok = np.flatnonzero(np.isfinite(t))
    return rng.choice(ok, size=shape).astype(np.uint8)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (16, 16, 16), (3, 32, 48), (17, 16, 128), (2, 48, 32)])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)], ids=["e4m3xe4m3", "e5m2xe4m3"])
def test_brute_force_triple_loop(m, n, k, fa, fb):
    rng = np.random.default_rng(m * 1000 + n * 10 + k)
    a = _rand_codes(rng, (m, k), fa)
    b = _rand_codes(rng, (n, k), fb)
    sa, sb = np.float32(0.75), np.float32(1.0 / 3.0)
    bias = rng.standard_normal(n).astype(np.float32)
    got = gemm_per_tensor(a, fa, sa, b, fb, sb, bias=bias, out="f32")
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += Fraction(decode(int(a[i, kk]), fa)) * Fraction(decode(int(b[j, kk]), fb))
            ref = float(acc) * float(sa) * float(sb) + float(bias[j])
            assert abs(got[i, j] - ref) <= 1e-5 * max(1.0, abs(ref)), (i, j)


def test_integer_operands_exact():
    """Integer-valued FP8 operands: the sum is an integer below 2^24, exact in any order."""
    rng = np.random.default_rng(1)
    ints = np.arange(-16, 17)
    codes = encode(ints.astype(np.float32), E4M3)
    assert (decode_table(E4M3)[codes] == ints).all()
    m, n, k = 32, 48, 256
    ia = rng.integers(0, len(ints), (m, k))
    ib = rng.integers(0, len(ints), (n, k))
    got = gemm_per_tensor(codes[ia], E4M3, 1.0, codes[ib], E4M3, 1.0, out="f32")
    ref = ints[ia].astype(np.int64) @ ints[ib].astype(np.int64).T
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def test_identity_operand():
    rng = np.random.default_rng(2)
    k = 64
    a = _rand_codes(rng, (16, k), E5M2)
    eye = np.where(np.eye(k, dtype=bool), 0x38, 0x00).astype(np.uint8)  # E4M3 1.0 = 0x38
    got = gemm_per_tensor(a, E5M2, 0.5, eye, E4M3, 4.0, out="f32")
    np.testing.assert_array_equal(got, (decode_table(E5M2)[a] * 2.0).astype(np.float32))


def test_bias_only():
    rng = np.random.default_rng(3)
    bias = rng.standard_normal(32).astype(np.float32)
    a = np.zeros((5, 16), dtype=np.uint8)
    b = _rand_codes(rng, (32, 16), E4M3)
    got = gemm_per_tensor(a, E4M3, 3.0, b, E4M3, 7.0, bias=bias, out="f32")
    np.testing.assert_array_equal(got, np.broadcast_to(bias, (5, 32)))
    got16 = gemm_per_tensor(a, E4M3, 3.0, b, E4M3, 7.0, bias=bias, out="bf16")
    ref16 = torch.from_numpy(bias).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got16, np.broadcast_to(ref16, (5, 32)))


def test_power_of_two_scale_linearity():
    rng = np.random.default_rng(4)
    a = _rand_codes(rng, (8, 32), E4M3)
    b = _rand_codes(rng, (16, 32), E4M3)
    d1 = gemm_per_tensor(a, E4M3, 0.3, b, E4M3, 1.7, out="f32")
    d2 = gemm_per_tensor(a, E4M3, 0.6, b, E4M3, 1.7, out="f32")
    np.testing.assert_array_equal(d2, 2 * d1)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 1e3,
        np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max, 1e-40, -1e-40], np.float32),
        # exact ties: low 16 bits 0x8000 with even and odd upper parts
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_round_bits(x), ref)
    nan = bf16_round_bits(np.array([np.nan], np.float32))
    assert np.isnan(bf16_bits_to_f32(nan)).all()


def test_mx_all_unit_scales_equal_per_tensor():
    rng = np.random.default_rng(6)
    a = _rand_codes(rng, (16, 96), E4M3)
    b = _rand_codes(rng, (32, 96), E4M3)
    ea = np.full((16, 3), 127, np.uint8)
    eb = np.full((32, 3), 127, np.uint8)
    bias = rng.standard_normal(32).astype(np.float32)
    np.testing.assert_array_equal(
        gemm_mx(a, ea, E4M3, b, eb, E4M3, bias=bias, out="f32"),
        gemm_per_tensor(a, E4M3, 1.0, b, E4M3, 1.0, bias=bias, out="f32"))


def test_mx_block_decomposition_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(20):
        k = 32 * int(rng.integers(1, 5))
        a = _rand_codes(rng, (1, k), E4M3)
        b = _rand_codes(rng, (1, k), E4M3)
        ea = rng.integers(100, 150, (1, k // 32)).astype(np.uint8)
        eb = rng.integers(100, 150, (1, k // 32)).astype(np.uint8)
        acc = Fraction(0)
        for blk in range(k // 32):
            dot = sum(Fraction(decode(int(a[0, i]), E4M3)) * Fraction(decode(int(b[0, i]), E4M3))
                      for i in range(blk * 32, blk * 32 + 32))
            acc += Fraction(2) ** (int(ea[0, blk]) - 127) * Fraction(2) ** (int(eb[0, blk]) - 127) * dot
        got = gemm_mx(a, ea, E4M3, b, eb, E4M3, out="f32")
        assert got[0, 0] == np.float32(float(acc))


def test_e8m0_values():
    assert e8m0_to_float(127) == 1.0
    assert e8m0_to_float(0) == 2.0 ** -127
    assert e8m0_to_float(254) == 2.0 ** 127


def test_bf16_gemm_brute_force():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((4, 40)).astype(np.float32)
    b = rng.standard_normal((6, 40)).astype(np.float32)
    ab = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bb = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = gemm_bf16(ab, bb, out="f32")
    af = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    bf = torch.from_numpy(b).to(torch.bfloat16).double().numpy()
    for i in range(4):
        for j in range(6):
            acc = sum(Fraction(float(af[i, kk])) * Fraction(float(bf[j, kk])) for kk in range(40))
            assert got[i, j] == np.float32(float(acc))


def test_rel_err_definition():
    r = np.array([1.0, -2.0, 1000.0])
    assert rel_err(r, r) == 0.0
    d = r + np.array([0.01, 0.0, 0.0])
    assert abs(rel_err(d, r) - 0.01) < 1e-12
    # near-zero reference uses the 1e-3 * max floor
    r2 = np.array([0.0, 1000.0])
    assert abs(rel_err(np.array([0.5, 1000.0]), r2) - 0.5) < 1e-12


def test_bias_grad_pins():
    """bias_grad against a Python double loop on a tiny input, the closed form of a
    rank-one dy (every row the same vector v: db = R v), and the gradient of the bias
    by finite differences of sum(y * dy) with y = x W^T + b (linear in b, so exact)."""
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((7, 5)).astype(np.float32)
    loop = [sum(float(dy[r, c]) for r in range(7)) for c in range(5)]
    np.testing.assert_allclose(bias_grad(dy), loop, rtol=0, atol=1e-12)
    v = rng.integers(-50, 50, 6).astype(np.float32)
    np.testing.assert_array_equal(bias_grad(np.tile(v, (13, 1))), 13.0 * v.astype(np.float64))
    x = rng.standard_normal((9, 4))
    w = rng.standard_normal((3, 4))
    b = rng.standard_normal(3)
    g = rng.standard_normal((9, 3))
    loss = lambda bb: float(np.sum((x @ w.T + bb) * g))  # noqa: E731
    fd = np.array([loss(b + np.eye(3)[c]) - loss(b) for c in range(3)])
    np.testing.assert_allclose(bias_grad(g), fd, rtol=1e-12, atol=1e-12)


def test_gemm_with_amax_brute_force_and_bf16_relation():
    """amax of the stored output, by a Python loop over the oracle's own output and, for
    bf16, the closed form bf16(max |d32|): rounding to bf16 is monotone in |d|, so the
    largest stored magnitude is the rounding of the largest fp32 one."""
    rng = np.random.default_rng(11)
    m, n, k = 9, 16, 32
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    b = rng.integers(0, 256, (n, k)).astype(np.uint8)
    a[a == 0x7F] = 0x7E
    a[a == 0xFF] = 0xFE
    b[(b & 0x7F) == 0x7F] = 0x38
    bias = rng.standard_normal(n).astype(np.float32)
    for out in ("bf16", "f32"):
        d, am = O.gemm_with_amax(a, O.E4M3, np.float32(0.5), b, O.E4M3, np.float32(0.25), bias=bias, out=out)
        ref = max(abs(float(v)) for v in d.reshape(-1))
        assert am == np.float32(ref)
    d32, am32 = O.gemm_with_amax(a, O.E4M3, np.float32(0.5), b, O.E4M3, np.float32(0.25), bias=bias, out="f32")
    _, am16 = O.gemm_with_amax(a, O.E4M3, np.float32(0.5), b, O.E4M3, np.float32(0.25), bias=bias, out="bf16")
    assert am16 == O.bf16_bits_to_f32(O.bf16_round_bits(np.array([am32], np.float32)))[0]


def test_gemm_with_amax_fp8_output_worked_by_hand():
    """FP8 output: the fp32 result cast with the given scale.  Integer operands 1 (0x38)
    and 2 (0x40): a row of k = 3 ones times a row of twos gives 6; scale 8 -> 48 =
    1.5 * 2^5, E4M3 field 5 + 7 = 12, mantissa 100 -> 0x64.  A result of 1000 at scale 1
    saturates to 0x7E while the amax keeps 1000 (the amax is of the values before the
    cast, as a separate cast of the fp32 output would record it)."""
    a = np.full((1, 16), 0x00, np.uint8)
    a[0, :3] = 0x38
    b = np.full((1, 16), 0x40, np.uint8)
    q, am = O.gemm_with_amax(a, O.E4M3, np.float32(1), b, O.E4M3, np.float32(1), out="fp8",
                             out_scale=np.float32(8), out_fmt=O.E4M3)
    assert q[0, 0] == 0x64 and am == 6.0
    bias = np.array([994.0], np.float32)
    q, am = O.gemm_with_amax(a, O.E4M3, np.float32(1), b, O.E4M3, np.float32(1), bias=bias, out="fp8",
                             out_scale=np.float32(1), out_fmt=O.E4M3)
    assert q[0, 0] == 0x7E and am == 1000.0
    # E5M2 output of -6 at scale 1/2: -3 = -1.5 * 2^1, field 1 + 15 = 16, mantissa 10 -> 0xC2
    q, am = O.gemm_with_amax(a, O.E4M3, np.float32(-1), b, O.E4M3, np.float32(1), out="fp8",
                             out_scale=np.float32(0.5), out_fmt=O.E5M2)
    assert q[0, 0] == 0xC2 and am == 6.0
