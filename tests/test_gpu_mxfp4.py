"""GPU parity of the MXFP4 path (E2M1 elements, E8M0 scale per 32) against the oracle.

The quantizer must match oracle.mxfp4 byte for byte (packed codes and scale codes),
row-wise and column-wise, fp32 and bf16 input, including the special blocks (all
zero, NaN, infinite, ties, fp32 subnormals).  The GEMM must lie within the error
bound of the matrix cores' arithmetic (gpu_util.fp8_gemm_error_bound: E2M1 products
are exact, so the bound is a superset) and within 1e-2 / 1e-3 normwise; with
integer-valued operands and unit scales (exact in any order) it must match bit for bit.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle as O
from oracle import mxfp4 as F
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth
from fp8_precision_transformer_amd.shapes import CODONFM_5B, layer_gemms

from gpu_util import DEV, check_fp8_gemm, dev_f32, dev_u8, host, input_pair

pytestmark = pytest.mark.gpu


def _seed(*key) -> int:
    return zlib.crc32(repr(key).encode()) & 0xFFFF


def _u8(*shape):
    return torch.full(shape, 0xAB, dtype=torch.uint8, device=DEV)  # poison: every byte must be written


def _quantize_gpu(xd, rows, cols, row=True, col=True):
    o = {}
    if row:
        o["q"], o["e"] = _u8(rows, cols // 2), _u8(rows, cols // 32)
    if col:
        o["qT"], o["eT"] = _u8(cols, rows // 2), _u8(cols, rows // 32)
    B.te_mxfp4_quantize(xd, o.get("q"), o.get("e"), o.get("qT"), o.get("eT"))
    return {k: host(v) for k, v in o.items()}


def _check_quant(got, x32, row=True, col=True):
    if row:
        q, e = F.mxfp4_quantize(x32)
        np.testing.assert_array_equal(got["e"], e)
        np.testing.assert_array_equal(got["q"], q)
    if col:
        qT, eT = F.mxfp4_quantize(np.ascontiguousarray(x32.T))
        np.testing.assert_array_equal(got["eT"], eT)
        np.testing.assert_array_equal(got["qT"], qT)


# fp32 input and bf16 input of ragged shape take 128 x 64 tiles (ragged in both
# directions, one tile, several); bf16 input of whole 128 x 128 tiles takes the
# persistent tile kernel (256 x 384, 1024 x 768)
QUANT_SHAPES = [(32, 32), (128, 64), (160, 96), (256, 384), (416, 1088), (1024, 768)]


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp4_quantize_parity(shape, dtype):
    r, c = shape
    x = synth.activations((r, c), 31, _seed(shape, dtype), 0, 0)
    xd, x32 = input_pair(x, dtype)
    _check_quant(_quantize_gpu(xd, r, c), x32)


@pytest.mark.parametrize("which", ["row", "col"])
@pytest.mark.parametrize("shape", [(192, 320), (256, 512)], ids=str)
def test_mxfp4_quantize_one_direction(which, shape):
    r, c = shape
    x = synth.grads((r, c), 31, 7, 0, 0)
    xd, x32 = input_pair(x, "bf16")
    row, col = which == "row", which == "col"
    _check_quant(_quantize_gpu(xd, r, c, row, col), x32, row, col)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp4_quantize_special_blocks(dtype):
    """All-zero, NaN, +-inf, ties at several block scales, subnormals, -0; NaN and
    infinities in the column-wise blocks too."""
    rng = np.random.default_rng(5)
    r, c = 128, 256
    x = (rng.standard_normal((r, c)) * 3).astype(np.float32)
    x[0, 0:32] = 0.0
    x[0, 32:64] = -0.0
    x[1, 5] = np.nan
    x[2, 40] = np.inf
    x[3, 70] = -np.inf
    # every midpoint between neighbouring E2M1 magnitudes, and values in (6, 8) that saturate
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 5.5, 0.1], np.float32)
    for i, e in enumerate([-3, 0, 4, 20, -60]):
        blk = np.zeros(32, np.float32)
        blk[0] = 7.0 * 2.0 ** e              # amax in [4, 8) * 2^e sets the block exponent to e
        blk[1:1 + len(mids)] = mids * 2.0 ** e * np.where(np.arange(len(mids)) % 2, -1, 1)
        blk[1 + len(mids):] = rng.uniform(-6, 6, 32 - 1 - len(mids)) * 2.0 ** e
        x[4 + i, 32 * (i % 8): 32 * (i % 8) + 32] = blk
    x[10, :32] = np.float32(2.0 ** -140) * np.arange(1, 33, dtype=np.float32)   # fp32 subnormals
    x[11, :32] = np.float32(3.0e38)
    x[12, 96:128] = -np.float32(1e-30)
    x[100, 200] = np.nan
    x[70:90, 150] = -np.inf
    xd, x32 = input_pair(x, dtype)
    got = _quantize_gpu(xd, r, c)
    _check_quant(got, x32)
    assert got["e"][1, 0] == 255 and got["e"][2, 1] == 254 and got["e"][0, 0] == 127
    assert got["eT"][200, 3] == 255 and got["eT"][150, 2] == 254


def test_mxfp4_quantize_bad_shapes():
    with pytest.raises(B.TEError):
        B.te_mxfp4_quantize(torch.zeros((32, 48), device=DEV), _u8(32, 24), _u8(32, 1))
    with pytest.raises(B.TEError):
        B.te_mxfp4_quantize(torch.zeros((48, 32), device=DEV), None, None, _u8(32, 24), _u8(32, 1))


def _mx4_operands(m, n, k, sd):
    xa = synth.activations((m, k), 37, sd, 0, 0)
    xb = synth.normal((n, k), 0.02, 37, sd, 1, 0)
    qa, ea = F.mxfp4_quantize(xa)
    qb, eb = F.mxfp4_quantize(xb)
    return qa, ea, qb, eb


def _out(m, n, odt):
    return torch.empty((m, n), dtype=torch.bfloat16 if odt == "bf16" else torch.float32, device=DEV)


# k % 256 == 0; m and n ragged against the 256 x 256 tile, several k stages
@pytest.mark.parametrize("mnk", [(32, 32, 256), (300, 272, 512), (1024, 768, 768), (256, 256, 4096),
                                 (520, 400, 1280), (1, 16, 256)], ids=str)
@pytest.mark.parametrize("odt", ["bf16", "f32"])
@pytest.mark.parametrize("bias", [None, "f32"])
def test_mxfp4_gemm_parity(mnk, odt, bias):
    m, n, k = mnk
    sd = _seed(mnk, odt, bias)
    qa, ea, qb, eb = _mx4_operands(m, n, k, sd)
    bias_h = synth.normal((n,), 0.02, 37, sd, 2, 0) if bias else None
    d = _out(m, n, odt)
    B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(ea), dev_u8(qb), "E2M1", dev_u8(eb), d,
                  bias=dev_f32(bias_h) if bias else None, gran=B.TE_GRAN_MX_BLOCK32)
    assert B.te_gemm_variant() == "gemm4_mxfp4_e2m1_e2m1_256x256_pingpong"
    ref = F.gemm_mxfp4(qa, ea, qb, eb, bias=bias_h, out=odt)
    check_fp8_gemm(host(d), ref, F.dequantize(qa, ea), F.dequantize(qb, eb), 1.0, odt)


@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_mxfp4_gemm_exact_integer_operands(odt):
    """Integer E2M1 values (0, +-1, +-2, +-3, +-4, +-6) at unit and power-of-two
    scales: every partial sum is exact, so the result is bit-exact."""
    rng = np.random.default_rng(3)
    m, n, k = 384, 320, 1024
    ints = np.array([0, 2, 4, 5, 6, 7, 8, 10, 12, 13, 14, 15], np.uint8)  # codes of integer values
    ca = ints[rng.integers(0, len(ints), (m, k))]
    cb = ints[rng.integers(0, len(ints), (n, k))]
    qa, qb = F.pack(ca), F.pack(cb)
    ea = np.full((m, k // 32), 127, np.uint8)
    eb = np.full((n, k // 32), 127, np.uint8)
    ea[0, :] = 130            # row 0 of A scaled by 2^3
    eb[:, 3] = 125            # block 3 of every B row scaled by 2^-2
    d = _out(m, n, odt)
    B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(ea), dev_u8(qb), "E2M1", dev_u8(eb), d, gran=B.TE_GRAN_MX_BLOCK32)
    np.testing.assert_array_equal(host(d), F.gemm_mxfp4(qa, ea, qb, eb, out=odt))


def test_mxfp4_quantize_then_gemm_end_to_end():
    """The GPU quantizer feeding the GPU GEMM equals the oracle's chain (the codes are
    bit-exact, so the GEMM is checked against the oracle on the oracle's codes)."""
    m, n, k = 512, 384, 1536
    xa = synth.activations((m, k), 41, 0, 0, 0)
    xb = synth.normal((n, k), 0.02, 41, 1, 0)
    da, a32 = input_pair(xa, "bf16")
    db, b32 = input_pair(xb, "bf16")
    qa, ea, qb, eb = _u8(m, k // 2), _u8(m, k // 32), _u8(n, k // 2), _u8(n, k // 32)
    B.te_mxfp4_quantize(da, qa, ea)
    B.te_mxfp4_quantize(db, qb, eb)
    d = _out(m, n, "bf16")
    B.te_fp8_gemm(qa, "E2M1", ea, qb, "E2M1", eb, d, gran=B.TE_GRAN_MX_BLOCK32)
    oqa, oea = F.mxfp4_quantize(a32)
    oqb, oeb = F.mxfp4_quantize(b32)
    np.testing.assert_array_equal(host(qa), oqa)
    np.testing.assert_array_equal(host(eb), oeb)
    ref = F.gemm_mxfp4(oqa, oea, oqb, oeb, out="bf16")
    check_fp8_gemm(host(d), ref, F.dequantize(oqa, oea), F.dequantize(oqb, oeb), 1.0, "bf16")


def test_mxfp4_gemm_rejects():
    a = _u8(256, 128)
    e = _u8(256, 8)
    d = _out(256, 256, "f32")
    with pytest.raises(B.TEError):   # k = 2 * 64 = 128 is not a multiple of 256
        B.te_fp8_gemm(_u8(256, 64), "E2M1", _u8(256, 4), _u8(256, 64), "E2M1", _u8(256, 4), d,
                      gran=B.TE_GRAN_MX_BLOCK32)
    with pytest.raises(B.TEError):   # E2M1 needs block scales
        B.te_fp8_gemm(a, "E2M1", e, a, "E2M1", e, d)
    with pytest.raises(ValueError):     # mixed E2M1 x E4M3: operand widths differ
        B.te_fp8_gemm(a, "E2M1", e, _u8(256, 256), "E4M3", e, d, gran=B.TE_GRAN_MX_BLOCK32)


@pytest.mark.parametrize("layout", ["rowmajor", "panel"])
@pytest.mark.parametrize("stage", ["fprop", "wgrad"])
def test_mxfp4_gemm_full_5b_shape_sampled(stage, layout):
    """A 5B-layer GEMM shape at full size, with row-major scales (the ping-pong kernel)
    and with panel-layout scales (the one-wave kernel the layer runs); the oracle checks
    64 rows x 256 columns."""
    g = {(x.weight, x.stage): x for x in layer_gemms(CODONFM_5B)}[("mlp_up", stage)]
    if g.k % 256:
        pytest.skip("k not a multiple of 256")
    rng = np.random.default_rng(_seed("mx4", stage))
    qa = rng.integers(0, 256, (g.m, g.k // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, (g.n, g.k // 2), dtype=np.uint8)
    ea = rng.integers(120, 134, (g.m, g.k // 32), dtype=np.uint8)
    eb = rng.integers(120, 134, (g.n, g.k // 32), dtype=np.uint8)
    d = _out(g.m, g.n, "bf16")
    if layout == "panel":
        B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(O.mx_scales_panel(ea)), dev_u8(qb), "E2M1",
                      dev_u8(O.mx_scales_panel(eb)), d, gran=B.TE_GRAN_MX_BLOCK32_PANEL)
        assert "panel_mfma16" in B.te_gemm_variant()
    else:
        B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(ea), dev_u8(qb), "E2M1", dev_u8(eb), d, gran=B.TE_GRAN_MX_BLOCK32)
    rows = np.sort(rng.choice(g.m, 64, replace=False))
    cols = np.sort(rng.choice(g.n, 256, replace=False))
    rows[-1], cols[-1] = g.m - 1, g.n - 1
    ref = F.gemm_mxfp4(qa[rows], ea[rows], qb[cols], eb[cols], out="bf16")
    check_fp8_gemm(host(d)[np.ix_(rows, cols)], ref, F.dequantize(qa[rows], ea[rows]),
                   F.dequantize(qb[cols], eb[cols]), 1.0, "bf16")


# the panel layout of the same scales (the one-wave kernel): bit-identical to the
# row-major MXFP4 GEMM (the ping-pong kernel)
@pytest.mark.parametrize("mnk", [(32, 32, 256), (300, 272, 512), (520, 400, 1280), (1, 16, 256),
                                 (256, 256, 4096)], ids=str)
def test_mxfp4_gemm_panel_scales_bit_identical(mnk):
    m, n, k = mnk
    sd = _seed(mnk, "panel")
    qa, ea, qb, eb = _mx4_operands(m, n, k, sd)
    pa, pb = O.mx_scales_panel(ea), O.mx_scales_panel(eb)
    for odt in ("bf16", "f32"):
        d1, d2 = _out(m, n, odt), _out(m, n, odt)
        B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(ea), dev_u8(qb), "E2M1", dev_u8(eb), d1,
                      gran=B.TE_GRAN_MX_BLOCK32)
        B.te_fp8_gemm(dev_u8(qa), "E2M1", dev_u8(pa), dev_u8(qb), "E2M1", dev_u8(pb), d2,
                      gran=B.TE_GRAN_MX_BLOCK32_PANEL)
        deep = "deepA" if m >= n else "deepB"  # the operand with more rows gets three stage slots
        assert B.te_gemm_variant() == f"gemm1w_mxfp4_e2m1_e2m1_256x256_panel_mfma16_{deep}"
        assert torch.equal(d1, d2), (mnk, odt)


@pytest.mark.parametrize("shape", [(128, 256), (384, 512), (256, 4096)], ids=str)
@pytest.mark.parametrize("which", ["row", "col", "both"])
def test_mxfp4_panel_scales(shape, which):
    R, C = shape
    x32 = synth.activations(shape, 38, R + C, 0, 0)
    xd, xh = input_pair(x32, "bf16")
    orow = torch.empty((R, C // 2), dtype=torch.uint8, device=DEV) if which != "col" else None
    srow = torch.empty(B.te_mx_scale_panel_bytes(R, C), dtype=torch.uint8, device=DEV) if which != "col" else None
    ocol = torch.empty((C, R // 2), dtype=torch.uint8, device=DEV) if which != "row" else None
    scol = torch.empty(B.te_mx_scale_panel_bytes(C, R), dtype=torch.uint8, device=DEV) if which != "row" else None
    B.te_mxfp4_quantize_panel(xd, orow, srow, ocol, scol)
    if orow is not None:
        q, e = F.mxfp4_quantize(xh)
        np.testing.assert_array_equal(host(orow), q)
        np.testing.assert_array_equal(O.mx_scales_from_panel(host(srow), R, C // 32), e)
    if ocol is not None:
        q, e = F.mxfp4_quantize(np.ascontiguousarray(xh.T))
        np.testing.assert_array_equal(host(ocol), q)
        np.testing.assert_array_equal(O.mx_scales_from_panel(host(scol), C, R // 32), e)
