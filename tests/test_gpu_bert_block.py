"""The BERT-base-shaped block ([FP8-intro] "HuggingFace BERT を例にした FP8 学習"; hidden
768, intermediate 3072, 32 x 128 = 4096 tokens) through the C ABI with per-tensor
current scaling: E4M3 activations and weights, E5M2 output gradients, the QKV
(768 -> 2304), attention-out (768 -> 768), MLP-up (768 -> 3072) and MLP-down
(3072 -> 768) layers, each with Fprop, Dgrad and Wgrad.

Every cast-transpose (row and transposed FP8 bytes, amax, scale, scale_inv) must
match the oracle bit for bit; every GEMM output is checked on 128 sampled rows
(all columns) against the oracle's exact sums within the matrix-core bound.
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth

from gpu_util import DEV, amax_ws, check_fp8_gemm, empty_f32, host, input_pair

pytestmark = pytest.mark.gpu

CFG = 2
M = 32 * 128
LAYERS = [("qkv", 768, 2304), ("attn_out", 768, 768), ("mlp_up", 768, 3072), ("mlp_down", 3072, 768)]
FMTS = {"E4M3": O.E4M3, "E5M2": O.E5M2}


def _quantize(x32, fmt):
    """te_cast_transpose (current scaling) of x, checked against the oracle; returns the
    device row/transposed bytes, the host reference bytes and scale_inv."""
    R, C = x32.shape
    xd, xh = input_pair(x32, "bf16")
    row = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    col = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    scale, sinv, am = empty_f32(), empty_f32(), empty_f32()
    B.te_cast_transpose(xd, fmt, B.TE_SCALE_CURRENT, 0, scale, sinv, am, row, col, workspace=amax_ws())
    f = FMTS[fmt]
    s = O.current_scale(O.amax(xh), f)
    ref_row, ref_col = O.cast_transpose(xh, s, f)
    assert host(am)[0] == O.amax(xh)
    assert host(scale)[0] == s and host(sinv)[0] == O.scale_inverse(s)
    np.testing.assert_array_equal(host(row), ref_row)
    np.testing.assert_array_equal(host(col), ref_col)
    return row, col, ref_row, ref_col, O.scale_inverse(s)


def _gemm_check(a_dev, a_ref, fa, sa, b_dev, b_ref, fb, sb, rng):
    m, n = a_ref.shape[0], b_ref.shape[0]
    d = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    one = lambda v: torch.tensor([v], dtype=torch.float32, device=DEV)  # noqa: E731
    B.te_fp8_gemm(a_dev, fa, one(float(sa)), b_dev, fb, one(float(sb)), d)
    rows = np.sort(rng.choice(m, 128, replace=False))
    rows[-1] = m - 1
    ref = O.gemm_per_tensor(a_ref[rows], FMTS[fa], sa, b_ref, FMTS[fb], sb, out="bf16")
    check_fp8_gemm(host(d)[rows], ref, O.decode_table(FMTS[fa])[a_ref[rows]], O.decode_table(FMTS[fb])[b_ref],
                   np.float64(sa) * np.float64(sb), "bf16")


@pytest.mark.parametrize("name,k,n", LAYERS, ids=[l[0] for l in LAYERS])
def test_bert_block_layer_current_scaling(name, k, n):
    li = [l[0] for l in LAYERS].index(name)
    x = synth.activations((M, k), CFG, li, synth.T_X, 0)
    w = synth.normal((n, k), 0.02, CFG, li, synth.T_W, 0)
    dy = synth.grads((M, n), CFG, li, synth.T_DY, 0)
    xr, xc, xr_h, xc_h, sx = _quantize(x, "E4M3")
    wr, wc, wr_h, wc_h, sw = _quantize(w, "E4M3")
    gr, gc, gr_h, gc_h, sg = _quantize(dy, "E5M2")
    rng = np.random.default_rng(li)
    _gemm_check(xr, xr_h, "E4M3", sx, wr, wr_h, "E4M3", sw, rng)   # Fprop  Y  = X  W^T
    _gemm_check(gr, gr_h, "E5M2", sg, wc, wc_h, "E4M3", sw, rng)   # Dgrad  dX = dY W
    _gemm_check(gc, gc_h, "E5M2", sg, xc, xc_h, "E4M3", sx, rng)   # Wgrad  dW = dY^T X
