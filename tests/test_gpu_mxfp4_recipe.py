"""GPU parity of te_mxfp4_quantize_recipe, the FP4 recipe's steps around the MXFP4
quantizer ([LP-opt] "実モデルにおける結果の解釈": random Hadamard transform of the Wgrad
inputs, stochastic rounding of gradients, 2D block scaling of weights), against
oracle/fp4_recipe.py: codes and E8M0 scales bit-exact (scales read back from the panel
layout with the oracle's pinned inverse), on ragged panel counts, on blocks holding NaN
and infinities, and on sampled columns of a CodonFM-5B-sized gradient; then the Wgrad
GEMM of transformed operands against the oracle's product of the same codes."""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth
from oracle.mxfp4 import dequantize, gemm_mxfp4, mxfp4_quantize

from gpu_util import DEV, check_fp8_gemm, dev_bf16_from_bits, host

pytestmark = pytest.mark.gpu

RHT, SR, TWO_D = B.TE_MX4_RHT, B.TE_MX4_SR, B.TE_MX4_2D


def _u8(*shape):
    return torch.empty(shape, dtype=torch.uint8, device=DEV)


def _run(xb_bits, flags, mask=0, seed=0, row=True, col=True):
    R, C = xb_bits.shape
    xd = dev_bf16_from_bits(xb_bits)
    orow, srow = (_u8(R, C // 2), _u8(B.te_mx_scale_panel_bytes(R, C))) if row else (None, None)
    ocol, scol = (_u8(C, R // 2), _u8(B.te_mx_scale_panel_bytes(C, R))) if col else (None, None)
    B.te_mxfp4_quantize_recipe(xd, flags, orow, srow, ocol, scol, sign_mask=mask, seed=seed)
    out = {}
    if row:
        out["row"] = (host(orow), O.mx_scales_from_panel(host(srow), R, C // 32))
    if col:
        out["col"] = (host(ocol), O.mx_scales_from_panel(host(scol), C, R // 32))
    return out


def _input(kind, shape, seed):
    x = synth.grads(shape, 51, seed, synth.T_DY, 0) if kind == "grad" else synth.activations(shape, 51, seed, 0, 0)
    bits = synth.to_bf16_bits(x)
    return bits, synth.bf16_bits_as_f32(bits)


SHAPES = [(128, 128), (256, 384), (384, 256), (512, 1024)]


@pytest.mark.parametrize("shape", SHAPES, ids=str)
@pytest.mark.parametrize("flags", [RHT, SR, RHT | SR], ids=["rht", "sr", "rht_sr"])
def test_recipe_row_and_column_copies_bit_exact(shape, flags):
    R, C = shape
    bits, xh = _input("grad", shape, R + 3 * C + flags)
    mask, seed = 0x9E37 ^ flags, 0x1234_5678_9ABC + R
    got = _run(bits, flags, mask, seed)
    # row copy: RNE or SR of x (the Hadamard transform is for the column copy only)
    ref_row = O.mxfp4_quantize_sr(xh, seed, 0) if flags & SR else mxfp4_quantize(xh)
    np.testing.assert_array_equal(got["row"][1], ref_row[1])
    np.testing.assert_array_equal(got["row"][0], ref_row[0])
    y = O.rht16_rows(xh, mask) if flags & RHT else xh
    yt = np.ascontiguousarray(y.T)
    ref_col = O.mxfp4_quantize_sr(yt, seed, 1) if flags & SR else mxfp4_quantize(yt)
    np.testing.assert_array_equal(got["col"][1], ref_col[1])
    np.testing.assert_array_equal(got["col"][0], ref_col[0])


@pytest.mark.parametrize("flags", [RHT, RHT | SR, SR], ids=["rht", "rht_sr", "sr"])
def test_recipe_one_copy_only(flags):
    bits, xh = _input("act", (256, 256), 7 + flags)
    mask, seed = 0x00F1, 99
    got = _run(bits, flags, mask, seed, row=False, col=True)
    y = O.rht16_rows(xh, mask) if flags & RHT else xh
    ref = O.mxfp4_quantize_sr(np.ascontiguousarray(y.T), seed, 1) if flags & SR else mxfp4_quantize(
        np.ascontiguousarray(y.T))
    np.testing.assert_array_equal(got["col"][0], ref[0])
    np.testing.assert_array_equal(got["col"][1], ref[1])
    if not flags & RHT:
        got = _run(bits, flags, mask, seed, row=True, col=False)
        ref = O.mxfp4_quantize_sr(xh, seed, 0)
        np.testing.assert_array_equal(got["row"][0], ref[0])


def test_recipe_nan_and_infinite_blocks():
    """A NaN spreads through its 16-row Hadamard group (every output of the group is NaN):
    those column blocks take scale code 255 and NaN elements go to +0; an infinity makes
    its group's outputs infinite or NaN; rows outside the groups are untouched."""
    bits, xh = _input("act", (128, 128), 77)
    xh = xh.copy()
    xh[5, 3] = np.nan
    xh[40, 9] = np.inf
    xh[70, 20] = -np.inf
    xh[100, 100] = np.nan
    bits = synth.to_bf16_bits(xh)
    xh = synth.bf16_bits_as_f32(bits)
    for flags in (RHT, RHT | SR, SR):
        got = _run(bits, flags, 0x0F0F, 5)
        y = O.rht16_rows(xh, 0x0F0F) if flags & RHT else xh
        ref = O.mxfp4_quantize_sr(np.ascontiguousarray(y.T), 5, 1) if flags & SR else mxfp4_quantize(
            np.ascontiguousarray(y.T))
        np.testing.assert_array_equal(got["col"][1], ref[1])
        np.testing.assert_array_equal(got["col"][0], ref[0])


@pytest.mark.parametrize("shape", [(128, 128), (256, 512), (640, 384)], ids=str)
def test_2d_weight_blocks_bit_exact(shape):
    R, C = shape
    w = synth.normal(shape, 0.02, 52, R + C, synth.T_W, 0)
    w[3, 7] = np.float32(0.5)  # one sub-tile with a large max
    bits = synth.to_bf16_bits(w)
    wh = synth.bf16_bits_as_f32(bits)
    got = _run(bits, TWO_D)
    qr, er, qc, ec = O.mxfp4_quantize_2d(wh)
    np.testing.assert_array_equal(got["row"][1], er)
    np.testing.assert_array_equal(got["row"][0], qr)
    np.testing.assert_array_equal(got["col"][1], ec)
    np.testing.assert_array_equal(got["col"][0], qc)
    # one copy per call (Fprop takes the row-wise copy, Dgrad the column-wise one)
    row_only = _run(bits, TWO_D, col=False)
    col_only = _run(bits, TWO_D, row=False)
    np.testing.assert_array_equal(row_only["row"][0], qr)
    np.testing.assert_array_equal(row_only["row"][1], er)
    np.testing.assert_array_equal(col_only["col"][0], qc)
    np.testing.assert_array_equal(col_only["col"][1], ec)


def test_recipe_full_5b_gradient_sampled_columns():
    """dY of the MLP-up GEMM, 15872 x 16384 bf16, Hadamard transform + stochastic rounding
    of the column copy (dY^T, the Wgrad operand): 16 sampled columns over all 15872 rows
    bit-exact, and the row copy's sampled rows."""
    R, C = 15872, 16384
    x = synth.grads((R, C), 53, 0, synth.T_DY, 0)
    bits = synth.to_bf16_bits(x)
    del x
    xh = synth.bf16_bits_as_f32(bits)
    mask, seed = 0xBEEF, 2024
    xd = dev_bf16_from_bits(bits)
    orow, srow = _u8(R, C // 2), _u8(B.te_mx_scale_panel_bytes(R, C))
    ocol, scol = _u8(C, R // 2), _u8(B.te_mx_scale_panel_bytes(C, R))
    B.te_mxfp4_quantize_recipe(xd, RHT | SR, orow, srow, ocol, scol, sign_mask=mask, seed=seed)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(0).choice(C, 16, replace=False))
    got_col = host(ocol[torch.as_tensor(cols, device=DEV)])
    sc = O.mx_scales_from_panel(host(scol), C, R // 32)
    y = O.rht16_rows(xh[:, cols], mask)  # the transform acts on each column separately
    for j, c in enumerate(cols):         # row c of the column copy (dY^T)
        q, e = O.mxfp4_quantize_sr(y[:, j].reshape(1, R), seed, 1, first_row=int(c))
        np.testing.assert_array_equal(got_col[j], q[0])
        np.testing.assert_array_equal(sc[c], e[0])
    rows = np.sort(np.random.default_rng(1).choice(R, 8, replace=False))
    got_row = host(orow[torch.as_tensor(rows, device=DEV)])
    for j, r in enumerate(rows):
        q, _ = O.mxfp4_quantize_sr(xh[r].reshape(1, C), seed, 0, first_row=int(r))
        np.testing.assert_array_equal(got_row[j], q[0])


def test_wgrad_of_transformed_operands():
    """Wgrad dW = dY^T X with both operands' column copies Hadamard-transformed with one
    sign mask (dY also stochastically rounded): the GEMM of the GPU's codes equals the
    oracle's product of the oracle's codes within the matrix-core bound, and stays close
    to the exact dW (the transform leaves the product unchanged; FP4 quantization error
    only)."""
    M, N, K = 512, 256, 384
    dyb, dyh = _input("grad", (M, N), 61)
    xb, xh = _input("act", (M, K), 62)
    mask, seed = 0x6A5D, 31337
    g = _run(dyb, RHT | SR, mask, seed, row=False)["col"]
    a = _run(xb, RHT, mask, 0, row=False)["col"]
    qg, eg = O.mxfp4_quantize_sr(np.ascontiguousarray(O.rht16_rows(dyh, mask).T), seed, 1)
    qa, ea = mxfp4_quantize(np.ascontiguousarray(O.rht16_rows(xh, mask).T))
    np.testing.assert_array_equal(g[0], qg)
    np.testing.assert_array_equal(a[0], qa)
    dw = torch.empty((N, K), dtype=torch.float32, device=DEV)
    sa = torch.from_numpy(O.mx_scales_panel(eg)).to(DEV)
    sb = torch.from_numpy(O.mx_scales_panel(ea)).to(DEV)
    B.te_fp8_gemm(torch.from_numpy(qg).to(DEV), "E2M1", sa, torch.from_numpy(qa).to(DEV), "E2M1", sb, dw,
                  gran=B.TE_GRAN_MX_BLOCK32_PANEL)
    ref = gemm_mxfp4(qg, eg, qa, ea, out="f32")
    check_fp8_gemm(host(dw), ref, dequantize(qg, eg), dequantize(qa, ea), 1.0, "f32", label="wgrad rht")
    exact = dyh.astype(np.float64).T @ xh.astype(np.float64)
    rel = np.linalg.norm(ref - exact) / np.linalg.norm(exact)
    assert rel < 0.2, rel  # FP4 quantization error of the product, not the transform's


@pytest.mark.parametrize("kw,status", [
    (dict(flags=TWO_D | SR), B.TE_ERR_ARG),
    (dict(flags=8), B.TE_ERR_ARG),
    (dict(flags=RHT, col=False), B.TE_ERR_ARG),
    (dict(flags=TWO_D, col=False, row=False), B.TE_ERR_NULL),
    (dict(flags=SR, shape=(128, 96)), B.TE_ERR_UNSUPPORTED),
])
def test_recipe_rejections(kw, status):
    shape = kw.pop("shape", (128, 128))
    col = kw.pop("col", True)
    row = kw.pop("row", True)
    R, C = shape
    x = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    orow, srow = (_u8(R, C // 2), _u8(max(B.te_mx_scale_panel_bytes(R, C), 16))) if row else (None, None)
    ocol, scol = (_u8(C, R // 2), _u8(max(B.te_mx_scale_panel_bytes(C, R), 16))) if col else (None, None)
    with pytest.raises(B.TEError) as ei:
        B.te_mxfp4_quantize_recipe(x, kw["flags"], orow, srow, ocol, scol)
    assert ei.value.status == status
