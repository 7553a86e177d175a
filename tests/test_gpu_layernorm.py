"""GPU parity of te_layernorm_fp8 (LayerNorm written straight as FP8 codes).

The kernel runs LayerNorm in fp32; the oracle in float64.  Every FP8 code must be one
that some value within the fp32 error bound of the exact y encodes to (encoding is
monotone, so the code lies between the codes of y - e and y + e), and nearly all
codes must equal the exact y's code.  mu, rsigma and amax lie within their fp32
bounds, and a second run gives identical bytes.  With current scaling the expected
codes come from the oracle alone: the amax can be anywhere in the oracle's interval
am +- e (e the largest fp32 error bound of y), so the scale lies between the scales
of its two ends, and every code must lie between the codes of the extreme products
of y +- e_y and those two scales; no value from the kernel enters the expected codes.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth

from gpu_util import DEV, amax_ws, empty_f32, host, input_pair, scalar

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bounds(x, g, y64, mu64, rs64, C):
    """fp32 error bounds (with a factor 2 of slack) for mu, rsigma and y."""
    ax = np.abs(x).mean(axis=1)
    e_mu = 2 * (C * U * ax + U * np.abs(mu64))
    d = x - mu64[:, None]
    var = (d * d).mean(axis=1)
    rel_var = 4 * C * U + 2 * e_mu * np.abs(d).mean(axis=1) / np.maximum(var, 1e-300) + 2 * e_mu ** 2 / np.maximum(var, 1e-300)
    rel_rs = 2 * (0.5 * rel_var + 2 * U)
    ad = np.abs(d) * rs64[:, None]
    e_y = 2 * (np.abs(g)[None, :] * (ad * (rel_rs[:, None] + 3 * U) + (e_mu * rs64)[:, None]) + U * np.abs(y64)) + 1e-30
    return e_mu, rel_rs, e_y


def _check(shape, xdt, pdt, fmt, mode, seed):
    R, C = shape
    f = O.E4M3 if fmt == "E4M3" else O.E5M2
    x32 = synth.activations(shape, 21, seed, 0, 0)
    xd, xh = input_pair(x32, xdt)
    g32 = 1.0 + synth.normal((C,), 0.1, 21, seed, 1, 0)
    b32 = synth.normal((C,), 0.1, 21, seed, 2, 0)
    gd, gh = input_pair(g32, pdt)
    bd, bh = input_pair(b32, pdt)
    eps = 1e-5
    outs = []
    for _ in range(2):
        out = torch.empty(shape, dtype=torch.uint8, device=DEV)
        mu, rs = empty_f32(R), empty_f32(R)
        am, sinv = empty_f32(), empty_f32()
        if mode == "delayed":
            scale = scalar(8.0)
            B.te_layernorm_fp8(xd, gd, bd, eps, fmt, B.TE_SCALE_DELAYED, 0, scale, sinv, am, out, mu, rs, workspace=amax_ws())
        else:
            scale = empty_f32()
            B.te_layernorm_fp8(xd, gd, bd, eps, fmt, B.TE_SCALE_CURRENT, 0, scale, sinv, am, out, mu, rs, workspace=amax_ws())
        outs.append((host(out), host(mu), host(rs), host(am)[0], host(scale)[0], host(sinv)[0]))
    (q, mu_g, rs_g, am_g, s_g, si_g), (q2, mu2, rs2, am2, _, _) = outs
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(mu_g, mu2)
    np.testing.assert_array_equal(rs_g, rs2)
    assert am_g == am2
    y64, mu64, rs64 = O.layernorm(xh, gh, bh, np.float32(eps))
    e_mu, rel_rs, e_y = _bounds(xh.astype(np.float64), gh.astype(np.float64), y64, mu64, rs64, C)
    assert np.all(np.abs(mu_g - mu64) <= e_mu)
    assert np.all(np.abs(rs_g - rs64) <= rel_rs * rs64)
    am64 = np.abs(y64).max()
    e_am = e_y.max()
    assert abs(am_g - am64) <= e_am, (am_g, am64)
    tab = O.decode_table(f)
    if mode == "current":
        # the scales of the two ends of the oracle's amax interval (scale falls as amax rises)
        s_lo = np.float64(O.current_scale(np.float32(am64 + e_am), f))
        s_hi = np.float64(O.current_scale(np.float32(max(am64 - e_am, 1e-30)), f))
        s_ref = np.float64(O.current_scale(np.float32(am64), f))
        assert s_lo <= s_g <= s_hi, (s_lo, s_g, s_hi)
    else:
        s_lo = s_hi = s_ref = np.float64(8.0)
        assert s_g == np.float32(8.0)
    assert si_g == O.scale_inverse(np.float32(s_g))
    # every code between the codes of the smallest and largest value y' * s' can take
    ylo, yhi = y64 - e_y, y64 + e_y
    lo = tab[O.encode(np.minimum(ylo * s_lo, ylo * s_hi).astype(np.float32), f)]
    hi = tab[O.encode(np.maximum(yhi * s_lo, yhi * s_hi).astype(np.float32), f)]
    got = tab[q]
    assert np.all((got >= lo) & (got <= hi)), int(np.sum(~((got >= lo) & (got <= hi))))
    exact = O.encode((y64 * s_ref).astype(np.float32), f)
    assert np.mean(q == exact) > 0.999


@pytest.mark.parametrize("shape", [(1, 16), (3, 768), (300, 4096), (4096, 768), (37, 1040)], ids=str)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["delayed", "current"])
def test_layernorm_fp8_parity(shape, xdt, mode):
    _check(shape, xdt, "f32", "E4M3", mode, zlib.crc32(repr((shape, xdt, mode)).encode()) & 0xFFFF)


@pytest.mark.parametrize("pdt", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["E4M3", "E5M2"])
def test_layernorm_fp8_params_and_formats(pdt, fmt):
    _check((512, 1024), "bf16", pdt, fmt, "current", 7)


def test_layernorm_fp8_5b_hidden_rows():
    """The CodonFM-5B hidden size (4096) on an eighth of the 15872 tokens."""
    _check((1984, 4096), "bf16", "bf16", "E4M3", "delayed", 11)


def test_layernorm_fp8_empty_and_bad_args():
    am, sinv = empty_f32(), empty_f32()
    am.fill_(5.0)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, device=DEV)
    out = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
    B.te_layernorm_fp8(x, g, g, 1e-5, "E4M3", B.TE_SCALE_DELAYED, 0, scalar(2.0), sinv, am, out, workspace=amax_ws())
    torch.cuda.synchronize()
    assert host(am)[0] == 0.0 and host(sinv)[0] == 0.5
    with pytest.raises(B.TEError):
        B.te_layernorm_fp8(torch.zeros((4, 40), device=DEV), torch.ones(40, device=DEV),
                           torch.ones(40, device=DEV), 1e-5, "E4M3", B.TE_SCALE_DELAYED, 0, scalar(1.0),
                           sinv, am, torch.empty((4, 40), dtype=torch.uint8, device=DEV), workspace=amax_ws())
