"""End-to-end runs of the Linear layer through the C ABI against the oracle.

The 768 -> 768 layer of [FP8-intro] "Transformer Engine の使い方" for 20 steps
of delayed scaling (history 16, max, margin 0, HYBRID): every step's FP8 bytes,
amax history, scale and scale_inv bit-exact; the bf16 output within the
matrix-core error bound of the oracle's exact product.
Also: backward (Dgrad/Wgrad) with delayed scaling after the autocast exit's
update, one scale update per format group, current scaling, the MXFP8 recipe, and
resume of the scaling state from a checkpoint.  GEMM outputs are checked with
``check_fp8_gemm`` (the matrix-core error model of ``tests/mfma_model.py``).
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_precision_transformer_amd import synth
from fp8_precision_transformer_amd.linear import Linear, fp8_autocast
from fp8_precision_transformer_amd.recipe import (DelayedScaling, Float8CurrentScaling, Format,
                                                  MXFP8BlockScaling)

from gpu_util import DEV, check_fp8_gemm, dev_f32, host

pytestmark = pytest.mark.gpu

CFG = 1


def _layer(seed=0):
    lin = Linear(768, 768, bias=True)
    w = synth.normal((768, 768), 0.02, CFG, 0, synth.T_W, seed)
    b = synth.normal((768,), 0.02, CFG, 0, synth.T_BIAS, seed)
    with torch.no_grad():
        lin.weight.copy_(dev_f32(w))
        lin.bias.copy_(dev_f32(b))
    return lin, w, b


def test_linear_768_delayed_20_steps_bit_exact_state():
    recipe = DelayedScaling(fp8_format=Format.HYBRID, amax_history_len=16, amax_compute_algo="max")
    lin, w, b = _layer()
    lin.keep_fp8_tensors = True
    sx = O.DelayedScalingState(O.E4M3, 16, "max", 0)
    sw = O.DelayedScalingState(O.E4M3, 16, "max", 0)
    for t in range(20):
        x = synth.uniform01((1024, 768), CFG, 0, synth.T_X, t)
        with torch.no_grad(), fp8_autocast(enabled=True, fp8_recipe=recipe):
            y = lin(dev_f32(x))
        xq, sxi = sx.cast(x)
        wq, swi = sw.cast(w)
        ref = O.gemm_per_tensor(xq, O.E4M3, sxi, wq, O.E4M3, swi, bias=b, out="bf16")
        sx.update()
        sw.update()
        np.testing.assert_array_equal(host(lin.last_fp8["xq"]), xq, err_msg=f"step {t} xq")
        np.testing.assert_array_equal(host(lin.last_fp8["wq"]), wq, err_msg=f"step {t} wq")
        st = lin.fp8_state_dict()
        np.testing.assert_array_equal(host(st["amax_history"])[0], sx.hist, err_msg=f"step {t}")
        np.testing.assert_array_equal(host(st["amax_history"])[1], sw.hist, err_msg=f"step {t}")
        assert host(st["scale"])[0] == sx.scale and host(st["scale"])[1] == sw.scale, t
        assert host(st["scale_inv"])[0] == sx.scale_inv and host(st["scale_inv"])[1] == sw.scale_inv, t
        check_fp8_gemm(host(y), ref, O.decode_table(O.E4M3)[xq], O.decode_table(O.E4M3)[wq],
                       np.float64(sxi) * np.float64(swi), "bf16")


def test_linear_state_resume_is_bit_identical():
    recipe = DelayedScaling()
    xs = [synth.uniform01((256, 768), CFG, 1, synth.T_X, t) for t in range(20)]
    lin, _, _ = _layer(1)
    outs = []
    for t in range(20):
        with torch.no_grad(), fp8_autocast(fp8_recipe=recipe):
            outs.append(lin(dev_f32(xs[t])).clone())
        if t == 9:
            saved = lin.fp8_state_dict()
    lin2, _, _ = _layer(1)
    lin2.load_fp8_state_dict(saved)
    for t in range(10, 20):
        with torch.no_grad(), fp8_autocast(fp8_recipe=recipe):
            y = lin2(dev_f32(xs[t]))
        assert torch.equal(y, outs[t]), t


@pytest.fixture
def fresh_pools():
    """Modules registered by earlier tests share the delayed-scaling pools; start empty."""
    from fp8_precision_transformer_amd import linear as linear_mod
    linear_mod._pools.clear()
    yield


def test_linear_backward_delayed_scaling_uses_the_forward_scales(fresh_pools):
    """Delayed scaling, forward inside fp8_autocast and backward after its exit (the exit's
    scale update rewrites the scaling state before backward runs): Dgrad and Wgrad must
    dequantize W^T and X^T with the scale_inv their forward casts used, and dY with the
    gradient group's scale.  Four steps against the oracle's delayed-scaling state machine;
    the gradient group updates at the first exit after a backward."""
    recipe = DelayedScaling(fp8_format=Format.HYBRID, amax_history_len=16, amax_compute_algo="max")
    lin, w, b = _layer(7)
    lin.keep_fp8_tensors = True
    M = 256
    sx = O.DelayedScalingState(O.E4M3, 16, "max", 0)
    sw = O.DelayedScalingState(O.E4M3, 16, "max", 0)
    sg = O.DelayedScalingState(O.E5M2, 16, "max", 0)
    t4, t5 = O.decode_table(O.E4M3), O.decode_table(O.E5M2)
    for t in range(4):
        x = synth.activations((M, 768), 7, 0, synth.T_X, t)
        dy = synth.grads((M, 768), 7, 0, synth.T_DY, t)
        xd = dev_f32(x).requires_grad_(True)
        lin.weight.grad = None
        with fp8_autocast(fp8_recipe=recipe):
            y = lin(xd)
        xq, sxi = sx.cast(x)
        wq, swi = sw.cast(w)
        sx.update()
        sw.update()
        if t > 0:
            sg.update()  # the exit after a backward updates the gradient group
        dyb = dev_f32(dy).to(torch.bfloat16)
        y.backward(dyb)
        dy_b = host(dyb)
        dyq, sgi = sg.cast(dy_b)
        np.testing.assert_array_equal(host(lin.last_fp8["xq"]), xq, err_msg=f"step {t}")
        st = lin.fp8_state_dict()
        np.testing.assert_array_equal(host(st["amax_history"])[2], sg.hist, err_msg=f"step {t} dY history")
        assert host(st["scale"])[2] == sg.scale and host(st["scale_inv"])[2] == sg.scale_inv, t
        ref_dx = O.gemm_per_tensor(dyq, O.E5M2, sgi, np.ascontiguousarray(wq.T), O.E4M3, swi, out="bf16")
        check_fp8_gemm(host(xd.grad), ref_dx, t5[dyq], t4[wq.T], np.float64(sgi) * np.float64(swi), "bf16")
        ref_dw = O.gemm_per_tensor(np.ascontiguousarray(dyq.T), O.E5M2, sgi, np.ascontiguousarray(xq.T), O.E4M3,
                                   sxi, out="f32")
        check_fp8_gemm(host(lin.weight.grad), ref_dw, t5[dyq.T], t4[xq.T], np.float64(sgi) * np.float64(sxi), "f32")


def test_autocast_exit_updates_each_format_group_once(monkeypatch, fresh_pools):
    """Three modules under one recipe: the exit issues one te_scale_update for the forward
    (E4M3) group of all of them, and, after a backward, one for the gradient group."""
    from fp8_precision_transformer_amd import binding as Bm
    recipe = DelayedScaling(amax_history_len=16)
    layers = [_layer(10 + i)[0] for i in range(3)]
    calls = []
    real = Bm.te_scale_update
    monkeypatch.setattr(Bm, "te_scale_update", lambda *a, **k: (calls.append(a[3]), real(*a, **k)))
    x = dev_f32(synth.activations((64, 768), 8, 0, synth.T_X, 0)).requires_grad_(True)
    with fp8_autocast(fp8_recipe=recipe):
        y = layers[2](layers[1](layers[0](x)))
    assert calls == ["E4M3"], calls
    y.float().sum().backward()
    calls.clear()
    with torch.no_grad(), fp8_autocast(fp8_recipe=recipe):
        layers[2](layers[1](layers[0](x)))
    assert calls == ["E4M3", "E5M2"], calls


def test_linear_backward_current_scaling():
    recipe = Float8CurrentScaling(fp8_format=Format.HYBRID)
    lin, w, b = _layer(2)
    lin.keep_fp8_tensors = True
    x = synth.activations((512, 768), 2, 0, synth.T_X, 0)
    dy = synth.grads((512, 768), 2, 0, synth.T_DY, 0)
    xd = dev_f32(x).requires_grad_(True)
    with fp8_autocast(fp8_recipe=recipe):
        y = lin(xd)
    y.backward(dev_f32(dy).to(torch.bfloat16))
    dy_b = host(dev_f32(dy).to(torch.bfloat16))
    sx = O.current_scale(O.amax(x), O.E4M3)
    swt = O.current_scale(O.amax(w), O.E4M3)
    sdy = O.current_scale(O.amax(dy_b), O.E5M2)
    xq, wq = O.scaled_cast(x, sx, O.E4M3), O.scaled_cast(w, swt, O.E4M3)
    dyq = O.scaled_cast(dy_b, sdy, O.E5M2)
    np.testing.assert_array_equal(host(lin.last_fp8["xq"]), xq)
    t4, t5 = O.decode_table(O.E4M3), O.decode_table(O.E5M2)
    ref_y = O.gemm_per_tensor(xq, O.E4M3, O.scale_inverse(sx), wq, O.E4M3, O.scale_inverse(swt), bias=b)
    check_fp8_gemm(host(y), ref_y, t4[xq], t4[wq],
                   np.float64(O.scale_inverse(sx)) * np.float64(O.scale_inverse(swt)), "bf16")
    ref_dx = O.gemm_per_tensor(dyq, O.E5M2, O.scale_inverse(sdy), np.ascontiguousarray(wq.T), O.E4M3,
                               O.scale_inverse(swt), out="bf16")
    # dx goes back to the input's fp32 dtype from the bf16 GEMM output (exact widening)
    check_fp8_gemm(host(xd.grad), ref_dx, t5[dyq], t4[wq.T],
                   np.float64(O.scale_inverse(sdy)) * np.float64(O.scale_inverse(swt)), "bf16")
    ref_dw = O.gemm_per_tensor(np.ascontiguousarray(dyq.T), O.E5M2, O.scale_inverse(sdy),
                               np.ascontiguousarray(xq.T), O.E4M3, O.scale_inverse(sx), out="f32")
    check_fp8_gemm(host(lin.weight.grad), ref_dw, t5[dyq.T], t4[xq.T],
                   np.float64(O.scale_inverse(sdy)) * np.float64(O.scale_inverse(sx)), "f32")
    # bias gradient from the dbias pass over dY: within the fp32 summation bound
    assert np.all(np.abs(host(lin.bias.grad).astype(np.float64) - O.bias_grad(dy_b)) <= _dbias_bound(dy_b))


def test_linear_mxfp8_forward():
    lin, w, b = _layer(3)
    x = synth.activations((256, 768), 3, 0, synth.T_X, 0)
    with torch.no_grad(), fp8_autocast(fp8_recipe=MXFP8BlockScaling()):
        y = lin(dev_f32(x))
    qa, ea = O.mxfp8_quantize(x)
    qb, eb = O.mxfp8_quantize(w)
    ref = O.gemm_mx(qa, ea, O.E4M3, qb, eb, O.E4M3, bias=b)
    t4 = O.decode_table(O.E4M3)
    check_fp8_gemm(host(y), ref, t4[qa] * np.repeat(O.e8m0_to_float(ea), 32, axis=1),
                   t4[qb] * np.repeat(O.e8m0_to_float(eb), 32, axis=1), 1.0, "bf16")


def _dbias_bound(dy):
    """recursive-summation bound of an fp32 column sum over R rows: R 2^-24 sum |dY|"""
    return dy.shape[0] * 2.0 ** -24 * np.abs(dy.astype(np.float64)).sum(0) + 1e-30


def test_linear_mxfp8_backward():
    """MXFP8 Fprop, Dgrad and Wgrad: the forward keeps the column-wise MX copies of x and
    W; dY is quantized row-wise and column-wise; the bias gradient comes from the dbias
    pass over dY."""
    lin, w, b = _layer(5)
    lin.keep_fp8_tensors = True
    M = 256
    x = synth.activations((M, 768), 5, 0, synth.T_X, 0)
    dy = synth.grads((M, 768), 5, 0, synth.T_DY, 0)
    xd = dev_f32(x).requires_grad_(True)
    with fp8_autocast(fp8_recipe=MXFP8BlockScaling()):
        y = lin(xd)
    y.backward(dev_f32(dy).to(torch.bfloat16))
    dy_b = host(dev_f32(dy).to(torch.bfloat16)).astype(np.float32)
    t4 = O.decode_table(O.E4M3)

    def val(q, e):
        return t4[q] * np.repeat(O.e8m0_to_float(e), 32, axis=1)

    qx, ex = O.mxfp8_quantize(x)
    qw, ew = O.mxfp8_quantize(w)
    qxT, exT = O.mxfp8_quantize(np.ascontiguousarray(x.T))
    qwT, ewT = O.mxfp8_quantize(np.ascontiguousarray(w.T))
    np.testing.assert_array_equal(host(lin.last_fp8["xqT"]), qxT)
    np.testing.assert_array_equal(host(lin.last_fp8["wsT"]), ewT)
    check_fp8_gemm(host(y), O.gemm_mx(qx, ex, O.E4M3, qw, ew, O.E4M3, bias=b), val(qx, ex), val(qw, ew), 1.0,
                   "bf16")
    qg, eg = O.mxfp8_quantize(dy_b)
    qgT, egT = O.mxfp8_quantize(np.ascontiguousarray(dy_b.T))
    ref_dx = O.gemm_mx(qg, eg, O.E4M3, qwT, ewT, O.E4M3, out="bf16")
    check_fp8_gemm(host(xd.grad), ref_dx, val(qg, eg), val(qwT, ewT), 1.0, "bf16")
    ref_dw = O.gemm_mx(qgT, egT, O.E4M3, qxT, exT, O.E4M3, out="f32")
    check_fp8_gemm(host(lin.weight.grad), ref_dw, val(qgT, egT), val(qxT, exT), 1.0, "f32")
    db_ref = O.bias_grad(dy_b)
    assert np.all(np.abs(host(lin.bias.grad).astype(np.float64) - db_ref) <= _dbias_bound(dy_b))


def test_linear_mxfp8_backward_needs_32_tokens():
    lin, _, _ = _layer(6)
    xd = dev_f32(synth.activations((48, 768), 6, 0, synth.T_X, 0)).requires_grad_(True)
    with pytest.raises(ValueError), fp8_autocast(fp8_recipe=MXFP8BlockScaling()):
        lin(xd)


def test_linear_outside_autocast_uses_bf16_gemm():
    lin, w, b = _layer(4)
    x = synth.activations((64, 768), 4, 0, synth.T_X, 0)
    with torch.no_grad():
        y = lin(dev_f32(x))
    xb = synth.to_bf16_bits(x)
    wb = synth.to_bf16_bits(w)
    ref = O.gemm_bf16(xb, wb, bias=b)
    assert O.rel_err(host(y), ref) <= 1e-2
