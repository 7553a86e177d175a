"""te_fp8_gemm_amax: the GEMM epilogue reduces the amax of its output and can write the
output as FP8 ([LP-opt] "実モデルにおける結果の解釈": the per-tensor amax is an extra
memory pass otherwise).

Parity against oracle.gemm_with_amax:
  * exact case (integer-valued FP8 operands, sums below 2^24, power-of-two scales):
    outputs, FP8 codes and amax bit-exact;
  * synthetic activations x weights: the output within the matrix-core error bound
    (mfma_model), the amax equal to max |D| of the stored output bit for bit and
    within the largest element bound of the oracle's amax; FP8 codes inside the code
    interval that the bound allows around the oracle's fp32 result (and > 99% equal to
    the oracle's codes), and equal to te_amax_cast of the fused kernel's own
    fp32 result with the same scale;
  * ragged tiles: rows and columns past the output do not enter the amax;
  * an empty output reports amax 0.
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth
from mfma_model import gemm_error_bound

from gpu_util import DEV, amax_ws, check_fp8_gemm, dev_f32, dev_u8, empty_f32, host, scalar

pytestmark = pytest.mark.gpu

FMT = {"E4M3": O.E4M3, "E5M2": O.E5M2}


def _int_codes(rng, shape, fmt):
    """Codes of small integers (|v| <= 8), exact in both formats."""
    v = rng.integers(-8, 9, size=shape).astype(np.float32)
    return O.encode(v, fmt)


@pytest.mark.parametrize("out", ["bf16", "f32", "E4M3", "E5M2"])
@pytest.mark.parametrize("fa,fb", [("E4M3", "E4M3"), ("E5M2", "E4M3")])
@pytest.mark.parametrize("shape", [(256, 256, 128), (300, 208, 96), (64, 512, 1024)], ids=str)
def test_fused_amax_exact_integer_operands(out, fa, fb, shape):
    m, n, k = shape
    rng = np.random.default_rng(m + n + k)
    a = _int_codes(rng, (m, k), FMT[fa])
    b = _int_codes(rng, (n, k), FMT[fb])
    bias = rng.integers(-64, 65, n).astype(np.float32)
    sa, sb = np.float32(0.5), np.float32(2.0 ** -3)
    ws = amax_ws()
    am = empty_f32()
    if out in ("bf16", "f32"):
        d = torch.empty((m, n), dtype=torch.bfloat16 if out == "bf16" else torch.float32, device=DEV)
        B.te_fp8_gemm_amax(dev_u8(a), fa, scalar(sa), dev_u8(b), fb, scalar(sb), d, am, ws, bias=dev_f32(bias))
        ref, ref_am = O.gemm_with_amax(a, FMT[fa], sa, b, FMT[fb], sb, bias=bias, out=out)
        np.testing.assert_array_equal(host(d), ref)
    else:
        d = torch.empty((m, n), dtype=torch.uint8, device=DEV)
        s_out = np.float32(0.25)
        si = empty_f32()
        B.te_fp8_gemm_amax_fp8(dev_u8(a), fa, scalar(sa), dev_u8(b), fb, scalar(sb), d, out, scalar(s_out), si, am,
                               ws, bias=dev_f32(bias))
        ref, ref_am = O.gemm_with_amax(a, FMT[fa], sa, b, FMT[fb], sb, bias=bias, out="fp8", out_scale=s_out,
                                       out_fmt=FMT[out])
        np.testing.assert_array_equal(host(d), ref)
        assert host(si)[0] == O.scale_inverse(s_out)
    assert host(am)[0] == ref_am


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(512, 768, 768), (1000, 1024, 512), (256, 4096, 2048)], ids=str)
def test_fused_amax_equals_max_of_stored_output(out, shape):
    m, n, k = shape
    x = synth.activations((m, k), 41, m, synth.T_X, 0)
    w = synth.normal((n, k), 0.02, 41, n, synth.T_W, 0)
    bias = synth.normal((n,), 0.02, 41, n, synth.T_BIAS, 0)
    sx, sw = O.current_scale(O.amax(x), O.E4M3), O.current_scale(O.amax(w), O.E4M3)
    xq, wq = O.scaled_cast(x, sx, O.E4M3), O.scaled_cast(w, sw, O.E4M3)
    six, siw = O.scale_inverse(sx), O.scale_inverse(sw)
    d = torch.empty((m, n), dtype=torch.bfloat16 if out == "bf16" else torch.float32, device=DEV)
    am = empty_f32()
    B.te_fp8_gemm_amax(dev_u8(xq), "E4M3", scalar(six), dev_u8(wq), "E4M3", scalar(siw), d, am, amax_ws(),
                       bias=dev_f32(bias))
    got = host(d)
    assert host(am)[0] == np.max(np.abs(got))  # the amax of what was stored, bit for bit
    ref, ref_am = O.gemm_with_amax(xq, O.E4M3, six, wq, O.E4M3, siw, bias=bias, out=out)
    t4 = O.decode_table(O.E4M3)
    scale = np.float64(six) * np.float64(siw)
    check_fp8_gemm(got, ref, t4[xq], t4[wq], scale, out, label="fused amax epilogue")
    bound = gemm_error_bound(t4[xq], t4[wq], scale, ref, out)
    assert abs(np.float64(host(am)[0]) - np.float64(ref_am)) <= bound.max()


@pytest.mark.parametrize("fmt", ["E4M3", "E5M2"])
def test_fused_fp8_output_codes(fmt):
    """FP8 output on synthetic data: every code within the interval the GEMM bound allows
    around the oracle's fp32 result, > 99% equal to the oracle's codes, and identical to
    te_amax_cast (delayed, same scale) of the same kernel's fp32 result; the amax equals
    max |fp32 result| of that run and is within the bound of the oracle's amax."""
    m, n, k = 768, 1024, 1024
    f = FMT[fmt]
    x = synth.activations((m, k), 42, 0, synth.T_X, 0)
    w = synth.normal((n, k), 0.02, 42, 0, synth.T_W, 0)
    sx, sw = O.current_scale(O.amax(x), O.E4M3), O.current_scale(O.amax(w), O.E4M3)
    xq, wq = O.scaled_cast(x, sx, O.E4M3), O.scaled_cast(w, sw, O.E4M3)
    six, siw = O.scale_inverse(sx), O.scale_inverse(sw)
    xd, wd = dev_u8(xq), dev_u8(wq)
    # a delayed-style scale (a power of two) at which the largest results saturate
    _, am_ref = O.gemm_with_amax(xq, O.E4M3, six, wq, O.E4M3, siw, out="f32")
    s_out = np.float32(2.0 ** np.ceil(np.log2(2.0 * f.max / float(am_ref))))
    ws = amax_ws()
    q = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    am, si = empty_f32(), empty_f32()
    B.te_fp8_gemm_amax_fp8(xd, "E4M3", scalar(six), wd, "E4M3", scalar(siw), q, fmt, scalar(s_out), si, am, ws)
    r32 = torch.empty((m, n), dtype=torch.float32, device=DEV)
    am32 = empty_f32()
    B.te_fp8_gemm_amax(xd, "E4M3", scalar(six), wd, "E4M3", scalar(siw), r32, am32, ws)
    got, r_gpu = host(q), host(r32)
    # the fused cast is the library's cast of the same fp32 values
    q2 = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    B.te_amax_cast(r32, fmt, B.TE_SCALE_DELAYED, 0, scalar(s_out), empty_f32(), empty_f32(), q2, workspace=ws)
    np.testing.assert_array_equal(got, host(q2))
    assert host(am)[0] == host(am32)[0] == np.max(np.abs(r_gpu))
    assert host(si)[0] == O.scale_inverse(s_out)
    # against the oracle alone
    ref_q, ref_am = O.gemm_with_amax(xq, O.E4M3, six, wq, O.E4M3, siw, out="fp8", out_scale=s_out, out_fmt=f)
    r_ref = O.gemm_per_tensor(xq, O.E4M3, six, wq, O.E4M3, siw, out="f32").astype(np.float64)
    t4 = O.decode_table(O.E4M3)
    e = gemm_error_bound(t4[xq], t4[wq], np.float64(six) * np.float64(siw), r_ref, "f32")
    tab = O.decode_table(f)
    lo = tab[O.encode(((r_ref - e) * np.float64(s_out)).astype(np.float32), f)]
    hi = tab[O.encode(((r_ref + e) * np.float64(s_out)).astype(np.float32), f)]
    v = tab[got]
    assert np.all((v >= lo) & (v <= hi))
    # statistical sanity check beside the interval (the parity bar): codes differ from the
    # oracle's only where the truncated matrix-core sum sits next to a rounding boundary
    assert np.mean(got == ref_q) > 0.99
    assert (got & 0x7F).max() == f.max_code  # some results saturate at this scale
    assert abs(np.float64(host(am)[0]) - np.float64(ref_am)) <= e.max()


def test_fused_amax_ignores_rows_and_columns_past_the_output():
    """m = 300 leaves 212 zero-filled rows in the second tile row, whose accumulators are 0
    and whose values would be the bias; with bias 1024 on column 3 and every real row's
    sum there -1024, the true amax is 0 and any leak shows as 1024."""
    m, n, k = 300, 208, 32
    a = np.full((m, k), 0x38, np.uint8)              # E4M3 1.0
    b = np.zeros((n, k), np.uint8)
    b[3, :] = O.encode(np.float32(-32.0), O.E4M3)    # 32 x (1 x -32) = -1024
    bias = np.zeros(n, np.float32)
    bias[3] = 1024.0
    d = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    am = empty_f32()
    B.te_fp8_gemm_amax(dev_u8(a), "E4M3", scalar(1.0), dev_u8(b), "E4M3", scalar(1.0), d, am, amax_ws(),
                       bias=dev_f32(bias))
    assert np.all(host(d) == 0.0)
    assert host(am)[0] == 0.0


def test_fused_amax_empty_output_and_rejections():
    am, si = empty_f32(), empty_f32()
    a = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
    b = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    d = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
    B.te_fp8_gemm_amax_fp8(a, "E4M3", scalar(1.0), b, "E4M3", scalar(1.0), d, "E4M3", scalar(4.0), si, am, amax_ws())
    assert host(am)[0] == 0.0 and host(si)[0] == 0.25
    with pytest.raises(B.TEError):  # no workspace
        B.te_fp8_gemm_amax(b, "E4M3", scalar(1.0), b, "E4M3", scalar(1.0),
                           torch.empty((64, 64), dtype=torch.bfloat16, device=DEV), am, None)
