"""GPU parity of the GEMMs (per-tensor FP8, MXFP8, BF16) against the CPU oracle.

FP8 and MXFP8: every element must lie within the error bound of the FP8 matrix
cores' own arithmetic (see gpu_util.fp8_gemm_error_bound: truncating 8-product
groups, fp32 accumulation, output rounding), and the normwise relative error
must be within 1e-2 (bf16 out) / 1e-3 (fp32 out).  BF16: max relative error
(oracle.rel_err) within 1e-2 / 1e-3.  Where the result is exact in any summation
order (integer-valued operands, |sum| < 2^24, power-of-two scales) the output
must match bit for bit, fp32 and bf16 alike.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth
from fp8_precision_transformer_amd.shapes import CODONFM_5B, layer_gemms

from gpu_util import DEV, check_fp8_gemm, dev_f32, dev_u8, host, scalar

pytestmark = pytest.mark.gpu

FMTS = {"E4M3": O.E4M3, "E5M2": O.E5M2}
TOL = {"bf16": 1e-2, "f32": 1e-3}


def _seed(*key) -> int:
    return zlib.crc32(repr(key).encode()) & 0xFFFF


def _quantized(shape, fmt, key, kind="act"):
    """Seeded FP8 codes of a realistic tensor: current-scaled cast of synthetic data."""
    x = synth.activations(shape, *key) if kind == "act" else synth.grads(shape, *key)
    f = FMTS[fmt]
    s = O.current_scale(O.amax(x), f)
    return O.scaled_cast(x, s, f), O.scale_inverse(s)


def _out(m, n, odt):
    return torch.empty((m, n), dtype=torch.bfloat16 if odt == "bf16" else torch.float32, device=DEV)


# k stages of 128 bytes: 1 (k 16, 128), 2 (k 256), 3 (k 272, ragged), 4 (k 400, ragged), 6, 8
GEMM_SHAPES = [(16, 16, 16), (1, 16, 128), (300, 272, 400), (256, 256, 128), (513, 512, 1024),
               (1024, 768, 768), (64, 2304, 768), (4096, 48, 272), (128, 64, 256)]


@pytest.mark.parametrize("mnk", GEMM_SHAPES, ids=str)
@pytest.mark.parametrize("fa,fb", [("E4M3", "E4M3"), ("E5M2", "E4M3"), ("E4M3", "E5M2"), ("E5M2", "E5M2")])
@pytest.mark.parametrize("odt", ["bf16", "f32"])
@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
def test_fp8_gemm_parity(mnk, fa, fb, odt, bias):
    m, n, k = mnk
    sd = _seed(mnk, fa, fb, odt, bias)
    a, sa = _quantized((m, k), fa, (11, sd, 0, 0), "act" if fa == "E4M3" else "grad")
    b, sb = _quantized((n, k), fb, (11, sd, 1, 0))
    bias_h = synth.normal((n,), 0.02, 11, sd, 2, 0) if bias else None
    if bias == "bf16":
        bits = synth.to_bf16_bits(bias_h)
        bias_d = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        bias_h = synth.bf16_bits_as_f32(bits)
    elif bias == "f32":
        bias_d = dev_f32(bias_h)
    else:
        bias_d = None
    d = _out(m, n, odt)
    B.te_fp8_gemm(dev_u8(a), fa, scalar(float(sa)), dev_u8(b), fb, scalar(float(sb)), d, bias=bias_d)
    ref = O.gemm_per_tensor(a, FMTS[fa], sa, b, FMTS[fb], sb, bias=bias_h, out=odt)
    check_fp8_gemm(host(d), ref, O.decode_table(FMTS[fa])[a], O.decode_table(FMTS[fb])[b],
                   np.float64(sa) * np.float64(sb), odt)


@pytest.mark.parametrize("mnk", [(64, 64, 128), (200, 96, 512), (512, 512, 2048), (300, 272, 400)], ids=str)
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_fp8_gemm_exact_integer_operands(mnk, odt):
    """Integer-valued FP8 operands with |sum| < 2^24: the accumulation is exact in any
    order, so the fp32 output, and its round-to-nearest-even bf16, match bit for bit."""
    m, n, k = mnk
    rng = np.random.default_rng(_seed(mnk))
    ints = np.arange(-16, 17)
    codes = O.encode(ints.astype(np.float32), O.E4M3)
    a = codes[rng.integers(0, len(ints), (m, k))]
    b = codes[rng.integers(0, len(ints), (n, k))]
    bias = (rng.integers(-64, 64, n) * 0.25).astype(np.float32)
    d = _out(m, n, odt)
    B.te_fp8_gemm(dev_u8(a), "E4M3", scalar(0.5), dev_u8(b), "E4M3", scalar(4.0), d, bias=dev_f32(bias))
    ref = O.gemm_per_tensor(a, O.E4M3, 0.5, b, O.E4M3, 4.0, bias=bias, out=odt)
    np.testing.assert_array_equal(host(d), ref)


def test_fp8_gemm_identity_and_bias_only():
    k = 256
    rng = np.random.default_rng(3)
    a = O.encode(rng.standard_normal((96, k)).astype(np.float32) * 10, O.E5M2)
    eye = np.where(np.eye(k, dtype=bool), 0x38, 0).astype(np.uint8)
    d = _out(96, k, "f32")
    B.te_fp8_gemm(dev_u8(a), "E5M2", scalar(0.25), dev_u8(eye), "E4M3", scalar(2.0), d)
    np.testing.assert_array_equal(host(d), (O.decode_table(O.E5M2)[a] * 0.5).astype(np.float32))
    bias = rng.standard_normal(k).astype(np.float32)
    z = np.zeros((33, k), np.uint8)
    d2 = _out(33, k, "f32")
    B.te_fp8_gemm(dev_u8(z), "E4M3", scalar(3.0), dev_u8(eye), "E4M3", scalar(5.0), d2, bias=dev_f32(bias))
    np.testing.assert_array_equal(host(d2), np.broadcast_to(bias, (33, k)))


@pytest.mark.parametrize("mnk", [(16, 16, 32), (300, 272, 416), (1024, 768, 768), (256, 512, 4096)], ids=str)
def test_bf16_gemm_parity(mnk):
    m, n, k = mnk
    sd = _seed(mnk)
    ab = synth.to_bf16_bits(synth.activations((m, k), 12, sd, 0, 0))
    bb = synth.to_bf16_bits(synth.normal((n, k), 0.02, 12, sd, 1, 0))
    ad = torch.from_numpy(ab.view(np.int16)).to(DEV).view(torch.bfloat16)
    bd = torch.from_numpy(bb.view(np.int16)).to(DEV).view(torch.bfloat16)
    for odt in ("bf16", "f32"):
        d = _out(m, n, odt)
        B.te_fp8_gemm(ad, "BF16", None, bd, "BF16", None, d)
        ref = O.gemm_bf16(ab, bb, out=odt)
        err = O.rel_err(host(d), ref)
        assert err <= TOL[odt], (odt, err)


# k % 128 == 0 takes the ping-pong kernel (scales loaded a dword per row and stage), other
# k the two-stage kernel; ragged m and n in both.  Ping-pong stage counts 1, 2, 3 (k 128,
# 256, 384: the prologue and the loop tail of the split load schedule), 5, 6 and 32.
@pytest.mark.parametrize("mnk", [(32, 32, 64), (300, 272, 416), (1024, 768, 768), (256, 256, 4096),
                                 (64, 128, 96), (520, 400, 640), (64, 64, 128), (200, 304, 256),
                                 (256, 512, 384)], ids=str)
@pytest.mark.parametrize("fa,fb", [("E4M3", "E4M3"), ("E5M2", "E4M3")])
def test_mx_gemm_parity(mnk, fa, fb):
    m, n, k = mnk
    sd = _seed(mnk, fa, fb)
    xa = synth.activations((m, k), 13, sd, 0, 0) if fa == "E4M3" else synth.grads((m, k), 13, sd, 0, 0)
    xb = synth.normal((n, k), 0.02, 13, sd, 1, 0)
    qa, ea = O.mxfp8_quantize(xa, FMTS[fa])
    qb, eb = O.mxfp8_quantize(xb, FMTS[fb])
    bias = synth.normal((n,), 0.02, 13, sd, 2, 0)
    for odt in ("bf16", "f32"):
        d = _out(m, n, odt)
        B.te_fp8_gemm(dev_u8(qa), fa, dev_u8(ea), dev_u8(qb), fb, dev_u8(eb), d, bias=dev_f32(bias),
                      gran=B.TE_GRAN_MX_BLOCK32)
        ref = O.gemm_mx(qa, ea, FMTS[fa], qb, eb, FMTS[fb], bias=bias, out=odt)
        av = O.decode_table(FMTS[fa])[qa] * np.repeat(O.e8m0_to_float(ea), 32, axis=1)
        bv = O.decode_table(FMTS[fb])[qb] * np.repeat(O.e8m0_to_float(eb), 32, axis=1)
        check_fp8_gemm(host(d), ref, av, bv, 1.0, odt)


def test_mx_gemm_unit_scales_equal_per_tensor_exactly():
    rng = np.random.default_rng(9)
    m, n, k = 128, 256, 512
    ints = np.arange(-16, 17)
    codes = O.encode(ints.astype(np.float32), O.E4M3)
    a = codes[rng.integers(0, len(ints), (m, k))]
    b = codes[rng.integers(0, len(ints), (n, k))]
    ea = np.full((m, k // 32), 127, np.uint8)
    eb = np.full((n, k // 32), 127, np.uint8)
    d1, d2 = _out(m, n, "f32"), _out(m, n, "f32")
    B.te_fp8_gemm(dev_u8(a), "E4M3", dev_u8(ea), dev_u8(b), "E4M3", dev_u8(eb), d1, gran=B.TE_GRAN_MX_BLOCK32)
    B.te_fp8_gemm(dev_u8(a), "E4M3", scalar(1.0), dev_u8(b), "E4M3", scalar(1.0), d2)
    assert torch.equal(d1, d2)
    # power-of-two block scales are exact as well: scale every block of row 0 by 2^3
    ea2 = ea.copy()
    ea2[0, :] = 130
    d3 = _out(m, n, "f32")
    B.te_fp8_gemm(dev_u8(a), "E4M3", dev_u8(ea2), dev_u8(b), "E4M3", dev_u8(eb), d3, gran=B.TE_GRAN_MX_BLOCK32)
    np.testing.assert_array_equal(host(d3), O.gemm_mx(a, ea2, O.E4M3, b, eb, O.E4M3, out="f32"))


@pytest.mark.parametrize("mnk", [(1024, 768, 768), (512, 512, 4096)], ids=str)
@pytest.mark.parametrize("fa", ["E4M3", "E5M2"])
@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_fp8_gemm_error_is_the_matrix_core_arithmetic(mnk, fa, odt):
    """Cross-check of where the element-wise gap to the oracle comes from: the vendor
    library's FP8 GEMM (torch._scaled_mm on hipBLASLt) on the same codes and scales runs
    on the same matrix-core instruction and lands on this library's result up to fp32
    summation order (f32 out) or one bf16 rounding step (bf16 out), while both differ
    from the oracle's exact sums by the truncating 8-product groups."""
    if not hasattr(torch, "_scaled_mm"):
        pytest.skip("torch._scaled_mm is not available")
    m, n, k = mnk
    sd = _seed(mnk, fa, odt, "lib")
    a, sa = _quantized((m, k), fa, (17, sd, 0, 0), "act" if fa == "E4M3" else "grad")
    b, sb = _quantized((n, k), "E4M3", (17, sd, 1, 0))
    td = {"E4M3": torch.float8_e4m3fn, "E5M2": torch.float8_e5m2}
    odt_t = torch.bfloat16 if odt == "bf16" else torch.float32
    d = _out(m, n, odt)
    B.te_fp8_gemm(dev_u8(a), fa, scalar(float(sa)), dev_u8(b), "E4M3", scalar(float(sb)), d)
    lib = torch._scaled_mm(dev_u8(a).view(td[fa]), dev_u8(b).view(td["E4M3"]).t(), scale_a=scalar(float(sa))[0],
                           scale_b=scalar(float(sb))[0], out_dtype=odt_t)
    ours, theirs = host(d).astype(np.float64), host(lib).astype(np.float64)
    ref = O.gemm_per_tensor(a, FMTS[fa], sa, b, O.E4M3, sb, out=odt)
    scale = float(np.abs(ref).max())
    if odt == "f32":
        assert np.abs(ours - theirs).max() <= 1e-5 * scale
    else:
        gap = np.abs(ours - theirs)
        assert np.all(gap <= 2.0 ** -7 * np.maximum(np.abs(ours), np.abs(theirs)) + 1e-5 * scale)
    # both sit equally far from the oracle (max relative error, denominator floored at 1e-3 max|r|)
    e_ours, e_lib = O.rel_err(ours, ref), O.rel_err(theirs, ref)
    assert abs(e_ours - e_lib) <= 0.1 * max(e_ours, e_lib) + 1e-4, (e_ours, e_lib)


def test_gemm_empty_and_bad_shape_raise():
    d = torch.empty((0, 16), dtype=torch.bfloat16, device=DEV)
    a = torch.empty((0, 32), dtype=torch.uint8, device=DEV)
    b = torch.zeros((16, 32), dtype=torch.uint8, device=DEV)
    B.te_fp8_gemm(a, "E4M3", scalar(1.0), b, "E4M3", scalar(1.0), d)  # m == 0: no launch, OK
    with pytest.raises(B.TEError):
        bad = torch.zeros((16, 24), dtype=torch.uint8, device=DEV)
        B.te_fp8_gemm(bad, "E4M3", scalar(1.0), bad, "E4M3", scalar(1.0),
                      torch.empty((16, 16), dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("stage", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("weight", ["qkv", "mlp_down"])
def test_fp8_gemm_full_5b_shape_sampled(stage, weight):
    """The 5B-layer shapes at full size, in the launch configuration the benchmark
    times; the oracle checks 96 sampled rows x 384 sampled columns."""
    g = {(x.weight, x.stage): x for x in layer_gemms(CODONFM_5B)}[(weight, stage)]
    fa = "E4M3" if stage == "fprop" else "E5M2"
    rng = np.random.default_rng(_seed(weight, stage))
    # random finite codes of mid-range magnitude with random signs (drawn as bytes, so the
    # full-size operands cost no host-side float work)
    def codes(shape, fmt):
        mag = rng.integers(0x18, 0x48, shape, dtype=np.uint8)
        return mag | (rng.integers(0, 2, shape, dtype=np.uint8) << 7)
    a = codes((g.m, g.k), fa)
    b = codes((g.n, g.k), "E4M3")
    d = _out(g.m, g.n, "bf16")
    B.te_fp8_gemm(dev_u8(a), fa, scalar(1 / 64), dev_u8(b), "E4M3", scalar(1 / 64), d)
    rows = np.sort(rng.choice(g.m, 96, replace=False))
    cols = np.sort(rng.choice(g.n, 384, replace=False))
    rows[-1] = g.m - 1
    cols[-1] = g.n - 1
    ref = O.gemm_per_tensor(a[rows], FMTS[fa], np.float32(1 / 64), b[cols], O.E4M3, np.float32(1 / 64), out="bf16")
    got = host(d)[np.ix_(rows, cols)]
    check_fp8_gemm(got, ref, O.decode_table(FMTS[fa])[a[rows]], O.decode_table(O.E4M3)[b[cols]],
                   (1 / 64) ** 2, "bf16")


@pytest.mark.parametrize("stage", ["fprop", "wgrad"])
def test_mx_gemm_panel_full_5b_shape_sampled(stage):
    """MXFP8 with panel-layout scales (the one-wave kernel the benchmark times) at a full
    5B-layer shape; the oracle checks 96 sampled rows x 384 sampled columns."""
    g = {(x.weight, x.stage): x for x in layer_gemms(CODONFM_5B)}[("qkv", stage)]
    fa = "E4M3" if stage == "fprop" else "E5M2"
    rng = np.random.default_rng(_seed("mxp", stage))
    def codes(shape):
        mag = rng.integers(0x18, 0x48, shape, dtype=np.uint8)
        return mag | (rng.integers(0, 2, shape, dtype=np.uint8) << 7)
    a, b = codes((g.m, g.k)), codes((g.n, g.k))
    ea = rng.integers(120, 134, (g.m, g.k // 32), dtype=np.uint8)
    eb = rng.integers(120, 134, (g.n, g.k // 32), dtype=np.uint8)
    d = _out(g.m, g.n, "bf16")
    B.te_fp8_gemm(dev_u8(a), fa, dev_u8(O.mx_scales_panel(ea)), dev_u8(b), "E4M3", dev_u8(O.mx_scales_panel(eb)), d,
                  gran=B.TE_GRAN_MX_BLOCK32_PANEL)
    assert "panel_mfma16" in B.te_gemm_variant()
    rows = np.sort(rng.choice(g.m, 96, replace=False))
    cols = np.sort(rng.choice(g.n, 384, replace=False))
    rows[-1], cols[-1] = g.m - 1, g.n - 1
    ref = O.gemm_mx(a[rows], ea[rows], FMTS[fa], b[cols], eb[cols], O.E4M3, out="bf16")
    av = O.decode_table(FMTS[fa])[a[rows]] * np.repeat(O.e8m0_to_float(ea[rows]), 32, axis=1)
    bv = O.decode_table(O.E4M3)[b[cols]] * np.repeat(O.e8m0_to_float(eb[cols]), 32, axis=1)
    check_fp8_gemm(host(d)[np.ix_(rows, cols)], ref, av, bv, 1.0, "bf16")


def test_dispatched_variant_is_the_requested_matrix_core_path():
    """te_gemm_variant names the kernel that ran: the FP8, MX and BF16 requests each take
    their own matrix-core path (no silent fallback to another precision); per-tensor FP8
    with k % 128 == 0 takes the one-wave kernel (the deep stage ring on A when m >= n),
    other k the ping-pong kernel; an MX GEMM whose k is not a multiple of 128 takes the
    two-stage kernel."""
    m, n = 256, 256
    rng = np.random.default_rng(3)
    for k in (256, 160):
        a = dev_u8(rng.integers(0, 0x30, (m, k), dtype=np.uint8))
        b = dev_u8(rng.integers(0, 0x30, (n, k), dtype=np.uint8))
        ea = dev_u8(np.full((m, k // 32), 127, np.uint8))
        eb = dev_u8(np.full((n, k // 32), 127, np.uint8))
        d = _out(m, n, "f32")
        for fa, fb in (("E4M3", "E4M3"), ("E5M2", "E4M3")):
            B.te_fp8_gemm(a, fa, scalar(1.0), b, fb, scalar(1.0), d)
            want = (f"gemm1w_fp8_{fa.lower()}_{fb.lower()}_256x256_mfma16_deepA" if k % 128 == 0
                    else f"gemm4_fp8_{fa.lower()}_{fb.lower()}_256x256_pingpong")
            assert B.te_gemm_variant() == want
            B.te_fp8_gemm(a, fa, ea, b, fb, eb, d, gran=B.TE_GRAN_MX_BLOCK32)
            want = (f"gemm4_mx_{fa.lower()}_{fb.lower()}_256x256_pingpong" if k % 128 == 0
                    else "gemm_mx_256x256_twostage")
            assert B.te_gemm_variant() == want
        xb = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
        wb = torch.zeros((n, k), dtype=torch.bfloat16, device=DEV)
        B.te_fp8_gemm(xb, "BF16", None, wb, "BF16", None, d)
        assert B.te_gemm_variant() == "gemm4_bf16_256x256_pingpong"
    torch.cuda.synchronize()


@pytest.mark.parametrize("mnk", [(300, 272, 416), (1024, 768, 768), (256, 512, 4096)], ids=str)
@pytest.mark.parametrize("gran", ["tensor", "mx"])
def test_gemm_accumulate_into_fp32(mnk, gran):
    """te_fp8_gemm_accumulate (Wgrad into an fp32 main gradient): D = fl32(D_old + r),
    twice in a row, within the matrix-core bound of D_old + r (+ r)."""
    m, n, k = mnk
    sd = _seed(mnk, gran, "acc")
    d_old = synth.normal((m, n), 1.0, 14, sd, 3, 0)
    bias = synth.normal((n,), 0.02, 14, sd, 2, 0)
    if gran == "tensor":
        a, sa = _quantized((m, k), "E5M2", (14, sd, 0, 0), "grad")
        b, sb = _quantized((n, k), "E4M3", (14, sd, 1, 0))
        args = (dev_u8(a), "E5M2", scalar(float(sa)), dev_u8(b), "E4M3", scalar(float(sb)))
        prod = O.gemm_per_tensor(a, O.E5M2, sa, b, O.E4M3, sb, bias=bias, out="f32").astype(np.float64)
        av, bv, sc = O.decode_table(O.E5M2)[a], O.decode_table(O.E4M3)[b], np.float64(sa) * np.float64(sb)
        kw = {}
    else:
        xa = synth.grads((m, k), 14, sd, 0, 0)
        xb = synth.normal((n, k), 0.02, 14, sd, 1, 0)
        a, ea = O.mxfp8_quantize(xa, O.E4M3)
        b, eb = O.mxfp8_quantize(xb, O.E4M3)
        args = (dev_u8(a), "E4M3", dev_u8(ea), dev_u8(b), "E4M3", dev_u8(eb))
        prod = O.gemm_mx(a, ea, O.E4M3, b, eb, O.E4M3, bias=bias, out="f32").astype(np.float64)
        av = O.decode_table(O.E4M3)[a] * np.repeat(O.e8m0_to_float(ea), 32, axis=1)
        bv = O.decode_table(O.E4M3)[b] * np.repeat(O.e8m0_to_float(eb), 32, axis=1)
        sc = 1.0
        kw = {"gran": B.TE_GRAN_MX_BLOCK32}
    d = dev_f32(d_old)
    for rep in (1, 2):
        B.te_fp8_gemm(*args, d, bias=dev_f32(bias), accumulate=True, **kw)
        ref = d_old.astype(np.float64) + rep * prod
        check_fp8_gemm(host(d), ref, av, bv, rep * sc, "f32")


def test_gemm_accumulate_exact_integer_operands():
    """Integer operands, power-of-two scales and an integer D_old: every sum is exact, so
    D_old + A.B^T comes out bit for bit; a bf16 D is rejected."""
    m, n, k = 200, 96, 512
    rng = np.random.default_rng(21)
    ints = np.arange(-16, 17)
    codes = O.encode(ints.astype(np.float32), O.E4M3)
    a = codes[rng.integers(0, len(ints), (m, k))]
    b = codes[rng.integers(0, len(ints), (n, k))]
    d_old = rng.integers(-1000, 1000, (m, n)).astype(np.float32)
    d = dev_f32(d_old)
    B.te_fp8_gemm(dev_u8(a), "E4M3", scalar(0.5), dev_u8(b), "E4M3", scalar(4.0), d, accumulate=True)
    ref = d_old + O.gemm_per_tensor(a, O.E4M3, 0.5, b, O.E4M3, 4.0, out="f32")
    np.testing.assert_array_equal(host(d), ref)
    with pytest.raises(ValueError):
        B.te_fp8_gemm(dev_u8(a), "E4M3", scalar(0.5), dev_u8(b), "E4M3", scalar(4.0), _out(m, n, "bf16"),
                      accumulate=True)


# Panel-layout scales (the oracle's permutation of the same E8M0 values): bit-identical to
# the row-major MX GEMM; stage counts 1 to 5 and 32, ragged m and n (padding rows of the
# last panel are read and never used)
@pytest.mark.parametrize("mnk", [(64, 64, 128), (200, 304, 256), (256, 512, 384), (300, 272, 512),
                                 (520, 400, 640), (1024, 768, 768), (256, 256, 4096)], ids=str)
@pytest.mark.parametrize("fa,fb", [("E4M3", "E4M3"), ("E5M2", "E4M3")])
def test_mx_gemm_panel_scales_bit_identical(mnk, fa, fb):
    m, n, k = mnk
    sd = _seed(mnk, fa, fb, "panel")
    xa = synth.activations((m, k), 14, sd, 0, 0) if fa == "E4M3" else synth.grads((m, k), 14, sd, 0, 0)
    xb = synth.normal((n, k), 0.02, 14, sd, 1, 0)
    qa, ea = O.mxfp8_quantize(xa, FMTS[fa])
    qb, eb = O.mxfp8_quantize(xb, FMTS[fb])
    pa, pb = O.mx_scales_panel(ea), O.mx_scales_panel(eb)
    assert pa.size == B.te_mx_scale_panel_bytes(m, k) and pb.size == B.te_mx_scale_panel_bytes(n, k)
    bias = synth.normal((n,), 0.02, 14, sd, 2, 0)
    for odt in ("bf16", "f32"):
        d1, d2 = _out(m, n, odt), _out(m, n, odt)
        B.te_fp8_gemm(dev_u8(qa), fa, dev_u8(ea), dev_u8(qb), fb, dev_u8(eb), d1, bias=dev_f32(bias),
                      gran=B.TE_GRAN_MX_BLOCK32)
        B.te_fp8_gemm(dev_u8(qa), fa, dev_u8(pa), dev_u8(qb), fb, dev_u8(pb), d2, bias=dev_f32(bias),
                      gran=B.TE_GRAN_MX_BLOCK32_PANEL)
        assert "_panel" in B.te_gemm_variant()
        assert torch.equal(d1, d2), (mnk, odt)
    ref = O.gemm_mx(qa, ea, FMTS[fa], qb, eb, FMTS[fb], bias=bias, out="f32")
    av = O.decode_table(FMTS[fa])[qa] * np.repeat(O.e8m0_to_float(ea), 32, axis=1)
    bv = O.decode_table(FMTS[fb])[qb] * np.repeat(O.e8m0_to_float(eb), 32, axis=1)
    check_fp8_gemm(host(d2), ref, av, bv, 1.0, "f32")


def test_mx_gemm_panel_rejects_k_not_multiple_of_128():
    m, n, k = 64, 64, 96
    a = torch.zeros((m, k), dtype=torch.uint8, device=DEV)
    s = torch.full((4096,), 127, dtype=torch.uint8, device=DEV)
    d = torch.empty((m, n), dtype=torch.float32, device=DEV)
    with pytest.raises(B.TEError):
        B.te_fp8_gemm(a, "E4M3", s, a, "E4M3", s, d, gran=B.TE_GRAN_MX_BLOCK32_PANEL)
    assert B.te_mx_scale_panel_bytes(300, 512) == 512 * 512 // 32
    assert B.te_mx_scale_panel_bytes(300, 96) == -1


# Split-K: k in `splits` ranges of whole stages, fp32 partial sums added in split order,
# then the epilogue.  Shapes with few tiles and long k (the Wgrad of small layers), a
# ragged k with one stage per split, ragged m and n; E5M2 x E4M3 as in Wgrad.
SPLITK_CASES = [((768, 768, 4096), 8), ((300, 272, 1024), 3), ((64, 2304, 768), 6), ((130, 48, 400), 4),
                ((2304, 768, 4096), 7), ((512, 512, 2048), 1)]


@pytest.mark.parametrize("mnk,splits", SPLITK_CASES, ids=str)
@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_fp8_gemm_splitk(mnk, splits, odt):
    m, n, k = mnk
    sd = _seed(mnk, splits, odt, "splitk")
    xa = synth.grads((m, k), 15, sd, 0, 0)
    xb = synth.activations((n, k), 15, sd, 1, 0)
    sa, sb = O.current_scale(O.amax(xa), O.E5M2), O.current_scale(O.amax(xb), O.E4M3)
    qa, qb = O.scaled_cast(xa, sa, O.E5M2), O.scaled_cast(xb, sb, O.E4M3)
    bias = synth.normal((n,), 0.02, 15, sd, 2, 0)
    ws = torch.empty(max(B.te_fp8_gemm_splitk_workspace_bytes(m, n, splits), 16), dtype=torch.uint8, device=DEV)
    d = _out(m, n, odt)
    args = (dev_u8(qa), "E5M2", scalar(O.scale_inverse(sa)), dev_u8(qb), "E4M3", scalar(O.scale_inverse(sb)))
    B.te_fp8_gemm_splitk(*args, d, splits, ws, bias=dev_f32(bias))
    if splits > 1:
        assert B.te_gemm_variant().endswith("_splitk")
    ref = O.gemm_per_tensor(qa, O.E5M2, O.scale_inverse(sa), qb, O.E4M3, O.scale_inverse(sb), bias=bias, out=odt)
    t4, t5 = O.decode_table(O.E4M3), O.decode_table(O.E5M2)
    check_fp8_gemm(host(d), ref, t5[qa], t4[qb],
                   np.float64(O.scale_inverse(sa)) * np.float64(O.scale_inverse(sb)), odt)
    d2 = _out(m, n, odt)  # deterministic: the split order is fixed
    B.te_fp8_gemm_splitk(*args, d2, splits, ws, bias=dev_f32(bias))
    assert torch.equal(d, d2)
    if splits == 1:  # one split is te_fp8_gemm, bit for bit
        d3 = _out(m, n, odt)
        B.te_fp8_gemm(*args, d3, bias=dev_f32(bias))
        assert torch.equal(d, d3)


def test_fp8_gemm_splitk_integer_operands_exact():
    """integer-valued codes with |sum| < 2^24: every partial and every split sum is exact,
    so the split-K result equals the exact product bit for bit"""
    rng = np.random.default_rng(21)
    m, n, k = 256, 128, 2048
    ints = np.arange(-8, 9)
    codes = O.encode(ints.astype(np.float32), O.E4M3)
    a = codes[rng.integers(0, len(ints), (m, k))]
    b = codes[rng.integers(0, len(ints), (n, k))]
    d = _out(m, n, "f32")
    ws = torch.empty(B.te_fp8_gemm_splitk_workspace_bytes(m, n, 5), dtype=torch.uint8, device=DEV)
    B.te_fp8_gemm_splitk(dev_u8(a), "E4M3", scalar(1.0), dev_u8(b), "E4M3", scalar(1.0), d, 5, ws)
    np.testing.assert_array_equal(host(d), O.gemm_per_tensor(a, O.E4M3, np.float32(1), b, O.E4M3, np.float32(1),
                                                             out="f32"))


def test_bf16_gemm_splitk():
    m, n, k = 768, 768, 3072
    a32 = synth.activations((m, k), 16, 0, 0, 0)
    b32 = synth.normal((n, k), 0.02, 16, 0, 1, 0)
    ab, bb = synth.to_bf16_bits(a32), synth.to_bf16_bits(b32)
    ad = torch.from_numpy(ab.view(np.int16)).to(DEV).view(torch.bfloat16)
    bd = torch.from_numpy(bb.view(np.int16)).to(DEV).view(torch.bfloat16)
    d = _out(m, n, "f32")
    ws = torch.empty(B.te_fp8_gemm_splitk_workspace_bytes(m, n, 6), dtype=torch.uint8, device=DEV)
    B.te_fp8_gemm_splitk(ad, "BF16", None, bd, "BF16", None, d, 6, ws)
    assert O.rel_err(host(d), O.gemm_bf16(ab, bb, out="f32")) <= 1e-3


def test_fp8_gemm_splitk_rejects():
    a = torch.zeros((64, 256), dtype=torch.uint8, device=DEV)
    one = scalar(1.0)
    d = _out(64, 64, "f32")
    ws = torch.empty(B.te_fp8_gemm_splitk_workspace_bytes(64, 64, 2), dtype=torch.uint8, device=DEV)
    for splits, w, status in ((3, ws, B.TE_ERR_ARG),          # 3 splits of 2 stages
                              (2, ws[:1024], B.TE_ERR_ARG),   # workspace too small
                              (2, ws[1:], B.TE_ERR_ALIGN),    # misaligned workspace
                              (0, ws, B.TE_ERR_ARG)):
        with pytest.raises(B.TEError) as e:
            B.te_fp8_gemm_splitk(a, "E4M3", one, a, "E4M3", one, d, splits, w)
        assert e.value.status == status, (splits, status)
