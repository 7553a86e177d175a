"""GEMM references: per-tensor scaled FP8, MXFP8 block-scaled, and BF16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout ("TN"): D[m, n] = sum_k A[m, k] * B[n, k]; both operands have the
reduction axis contiguous.  Fprop is D = X W^T; Dgrad feeds dY and W^T; Wgrad
feeds dY^T and X^T ([LP-opt] "autocast モードの使用と事前量子化の比較": the
three GEMMs of each linear layer are benchmarked separately).

[FP8-intro] "FP8 Training について": the FP8 GEMM runs on FP8 tensor cores with
high-precision master weights; [FP8-intro] "Transformer Engine の使い方":
``te.Linear(768, 768, bias=True)`` -- a bias is added to the output.

Readings taken where the pages are silent:
  * accumulation: every FP8 x FP8 product is exact; the oracle sums them in
    float64 and rounds once to fp32 ("fp32-accumulated" read as an fp32 result
    of the exact sum, so the reference does not depend on summation order);
  * epilogue: d = fl32(fl32(acc * a_scale_inv) * b_scale_inv), then
    fl32(d + bias) with bias widened to fp32, then round-to-nearest-even to
    bf16 (or kept as fp32);
  * MXFP8: acc = sum over 32-blocks of 2^(ea-127) * 2^(eb-127) * (block dot
    product), all exact in float64, rounded once to fp32; bias as above.

  * bias gradient: the backward of y = x W^T + b gives db[c] = sum over rows
    of dy[r, c]; the oracle returns that sum in float64 (exact to float64
    rounding), and a GPU sum in fp32 is held to the fp32 summation bound.
  * amax of a GEMM output ([LP-opt] "実モデルにおける結果の解釈": the per-tensor
    amax costs an extra memory pass; [FP8-intro] "FP8 Training について": every
    tensor that is cast to FP8 carries its own scale, the next layer's input
    included): the amax of the tensor as stored (bf16 or fp32 output), or, when
    the output itself is written as FP8 with a given scale (delayed scaling of the
    next layer's input), of the fp32 values before that cast, which is the value a
    separate cast of the fp32 output would record.

Pins (tests/test_oracle_gemm.py): brute-force triple loop on tiny shapes,
integer-valued operands (exact in any order), identity operand, bias-only,
power-of-two scale linearity, MX with all codes 127 equal to per-tensor,
and the bf16 rounding against PyTorch's CPU conversion.  The tolerance
denominator of ``rel_err`` is a reading (parity unpinned for that choice).
"""

from __future__ import annotations

import numpy as np

from .formats import FP8Format, decode_table
from .quantize import amax, e8m0_to_float, scaled_cast


def bf16_round_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (NaN -> quiet NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    sign = ((u >> 16) & 0x8000).astype(np.uint16)
    return np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _decode(codes, fmt: FP8Format) -> np.ndarray:
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def _epilogue(acc32: np.ndarray, bias, out: str) -> np.ndarray:
    d = acc32
    if bias is not None:
        d = (d + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    if out == "f32":
        return d
    if out == "bf16":
        return bf16_bits_to_f32(bf16_round_bits(d))
    raise ValueError(out)


def gemm_per_tensor(a_codes, a_fmt: FP8Format, a_scale_inv, b_codes, b_fmt: FP8Format,
                    b_scale_inv, bias=None, out: str = "bf16") -> np.ndarray:
    """D = (A_q . B_q^T) * a_scale_inv * b_scale_inv + bias, per the reading above.

    Returns fp32 values (bf16-representable when out == "bf16").
    """
    a = _decode(a_codes, a_fmt)
    b = _decode(b_codes, b_fmt)
    acc = (a @ b.T).astype(np.float32)  # exact products, float64 sum, one rounding to fp32
    with np.errstate(over="ignore", invalid="ignore"):
        d = (acc * np.float32(a_scale_inv)).astype(np.float32)
        d = (d * np.float32(b_scale_inv)).astype(np.float32)
    return _epilogue(d, bias, out)


def gemm_with_amax(a_codes, a_fmt: FP8Format, a_scale_inv, b_codes, b_fmt: FP8Format, b_scale_inv,
                   bias=None, out: str = "bf16", out_scale=None, out_fmt: FP8Format = None):
    """The per-tensor GEMM of ``gemm_per_tensor`` together with the amax of its output.

    out "bf16" / "f32": returns (d, amax) with amax = max |d| over the stored values.
    out "fp8": the fp32 result d32 (bias added) is cast with ``out_scale`` to ``out_fmt``
    exactly as ``scaled_cast`` casts any tensor; returns (codes, amax = max |d32|).
    """
    if out in ("bf16", "f32"):
        d = gemm_per_tensor(a_codes, a_fmt, a_scale_inv, b_codes, b_fmt, b_scale_inv, bias=bias, out=out)
        return d, amax(d)
    if out != "fp8":
        raise ValueError(out)
    d32 = gemm_per_tensor(a_codes, a_fmt, a_scale_inv, b_codes, b_fmt, b_scale_inv, bias=bias, out="f32")
    return scaled_cast(d32, out_scale, out_fmt), amax(d32)


def gemm_mx(a_codes, a_e8m0, a_fmt: FP8Format, b_codes, b_e8m0, b_fmt: FP8Format,
            bias=None, out: str = "bf16", block: int = 32) -> np.ndarray:
    """MXFP8 GEMM: per-block power-of-two scales applied inside the K sum."""
    a = _decode(a_codes, a_fmt)
    b = _decode(b_codes, b_fmt)
    M, K = a.shape
    N = b.shape[0]
    sa = np.repeat(e8m0_to_float(a_e8m0), block, axis=1)  # [M, K]
    sb = np.repeat(e8m0_to_float(b_e8m0), block, axis=1)  # [N, K]
    acc = ((a * sa) @ (b * sb).T).astype(np.float32)  # power-of-two scaling is exact in float64
    return _epilogue(acc, bias, out)


def gemm_bf16(a_bits, b_bits, bias=None, out: str = "bf16") -> np.ndarray:
    """BF16 comparison GEMM: exact products of bf16 inputs, float64 sum, fp32 result."""
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    b = bf16_bits_to_f32(b_bits).astype(np.float64)
    acc = (a @ b.T).astype(np.float32)
    return _epilogue(acc, bias, out)


def bias_grad(dy) -> np.ndarray:
    """Bias gradient of y = x W^T + b ([FP8-intro] "Transformer Engine の使い方",
    te.Linear with bias): db[c] = sum_r dy[r, c], summed in float64."""
    return np.asarray(dy, dtype=np.float64).sum(axis=0)


def rel_err(d, r) -> float:
    """max_i |d_i - r_i| / max(|r_i|, 1e-3 * max_j |r_j|)  (floor avoids near-zero blow-up)."""
    d = np.asarray(d, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    floor = 1e-3 * np.max(np.abs(r))
    den = np.maximum(np.abs(r), floor)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(d - r) / den))
