"""The 24-layer sweep of the MXFP8 workload ([LP-opt] "autocast モードの使用と事前量子化の
比較" MXFP8 comparison, sized down for the oracle): 24 independent weight sets, 16
training-like steps, the input growing x1.05 per step so the scales move every step.

Per-tensor delayed scaling (E4M3, history 16, max): every layer's X and W are cast
with the scale of the previous update, amax lands in history slot 0, and one
te_scale_update launch refreshes all 48 tensors; FP8 bytes, history, scale and
scale_inv must match the oracle bit for bit at every step.  MXFP8: every layer's X
quantized row-wise and column-wise at every step, codes and E8M0 scales bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import binding as B
from fp8_precision_transformer_amd import synth

from gpu_util import DEV, amax_ws, dev_bf16_from_bits, host

pytestmark = pytest.mark.gpu

CFG = 5
LAYERS, STEPS = 24, 16
M, K, N = 128, 256, 256


def _x(layer, step):
    """bf16 bits and exact fp32 values of layer `layer`'s input at `step` (fresh sample x 1.05^step)."""
    x = synth.activations((M, K), CFG, layer, synth.T_X, step) * np.float32(1.05 ** step)
    bits = synth.to_bf16_bits(x.astype(np.float32))
    return bits, synth.bf16_bits_as_f32(bits)


def test_delayed_sweep_24_layers_16_steps_drift():
    ws = [synth.normal((N, K), 0.02, CFG, l, synth.T_W, 0) for l in range(LAYERS)]
    wd = [torch.from_numpy(w).to(DEV) for w in ws]
    T = 2 * LAYERS  # tensor 2l = X of layer l, 2l+1 = W of layer l
    hist = torch.zeros((T, 16), dtype=torch.float32, device=DEV)
    scale = torch.ones(T, dtype=torch.float32, device=DEV)
    sinv = torch.ones(T, dtype=torch.float32, device=DEV)
    ref = [O.DelayedScalingState(O.E4M3, 16, "max", 0) for _ in range(T)]
    outs = [torch.empty((M, K), dtype=torch.uint8, device=DEV) for _ in range(LAYERS)]
    wouts = [torch.empty((N, K), dtype=torch.uint8, device=DEV) for _ in range(LAYERS)]
    for t in range(STEPS):
        xs = [_x(l, t) for l in range(LAYERS)]
        for l in range(LAYERS):
            xd = dev_bf16_from_bits(xs[l][0])
            B.te_amax_cast(xd, "E4M3", B.TE_SCALE_DELAYED, 0, scale[2 * l:2 * l + 1], sinv[2 * l:2 * l + 1],
                           hist[2 * l, 0:1], outs[l], workspace=amax_ws())
            B.te_amax_cast(wd[l], "E4M3", B.TE_SCALE_DELAYED, 0, scale[2 * l + 1:2 * l + 2],
                           sinv[2 * l + 1:2 * l + 2], hist[2 * l + 1, 0:1], wouts[l], workspace=amax_ws())
        got_hist_pre = host(hist)
        for l in range(LAYERS):
            xq, _ = ref[2 * l].cast(xs[l][1])
            wq, _ = ref[2 * l + 1].cast(ws[l])
            np.testing.assert_array_equal(host(outs[l]), xq, err_msg=f"step {t} layer {l} x")
            np.testing.assert_array_equal(host(wouts[l]), wq, err_msg=f"step {t} layer {l} w")
            assert got_hist_pre[2 * l, 0] == ref[2 * l].hist[0], (t, l)
        B.te_scale_update(hist, scale, sinv, "E4M3", B.TE_AMAX_MAX, 0)
        for r in ref:
            r.update()
        h, sc, si = host(hist), host(scale), host(sinv)
        for i, r in enumerate(ref):
            np.testing.assert_array_equal(h[i], r.hist, err_msg=f"step {t} tensor {i}")
            assert sc[i] == r.scale and si[i] == r.scale_inv, (t, i)
    # the drift keeps moving the X scales: the last scale is below the first nonzero one
    assert ref[0].scale < O.E4M3.max / O.amax(_x(0, 0)[1])


def test_mxfp8_sweep_24_layers_16_steps_drift():
    orow = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    srow = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    ocol = torch.empty((K, M), dtype=torch.uint8, device=DEV)
    scol = torch.empty((K, M // 32), dtype=torch.uint8, device=DEV)
    mean_codes = []
    for t in range(STEPS):
        codes_t = []
        for l in range(LAYERS):
            bits, xh = _x(l, t)
            B.te_mxfp8_quantize(dev_bf16_from_bits(bits), "E4M3", orow, srow, ocol, scol)
            q, e = O.mxfp8_quantize(xh, O.E4M3)
            qc, ec = O.mxfp8_quantize(np.ascontiguousarray(xh.T), O.E4M3)
            np.testing.assert_array_equal(host(orow), q, err_msg=f"step {t} layer {l} row codes")
            np.testing.assert_array_equal(host(srow), e, err_msg=f"step {t} layer {l} row scales")
            np.testing.assert_array_equal(host(ocol), qc, err_msg=f"step {t} layer {l} col codes")
            np.testing.assert_array_equal(host(scol), ec, err_msg=f"step {t} layer {l} col scales")
            codes_t.append(e.astype(np.float64).mean())
        mean_codes.append(np.mean(codes_t))
    # the shared exponents follow the drift: about +log2(1.05) per step on average
    slope = np.polyfit(np.arange(STEPS), mean_codes, 1)[0]
    assert 0.04 < slope < 0.10, slope
