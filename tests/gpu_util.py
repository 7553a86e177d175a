"""Helpers for the GPU parity tests: device tensors from host arrays, host copies back."""

import numpy as np
import torch

from fp8_precision_transformer_amd import synth

DEV = "cuda:0"


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_as_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def scalar(v) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def empty_f32(n=1) -> torch.Tensor:
    return torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)


def input_pair(x32: np.ndarray, dtype: str):
    """(device tensor, exact fp32 host values the oracle sees) for bf16 or fp32 input."""
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x32)
        return dev_bf16_from_bits(bits), synth.bf16_bits_as_f32(bits)
    return dev_f32(x32), np.ascontiguousarray(x32, dtype=np.float32)


def nan_aware_equal(got: np.ndarray, ref: np.ndarray, decode_tbl: np.ndarray):
    """Bytes equal, except that any NaN code is accepted where the oracle gives a NaN code."""
    ref_nan = np.isnan(decode_tbl[ref])
    got_nan = np.isnan(decode_tbl[got])
    bad = (~ref_nan & (got != ref)) | (ref_nan & ~got_nan)
    return int(bad.sum()), np.flatnonzero(bad.reshape(-1))[:10]


# --- FP8 matrix-core arithmetic, measured on gfx950 through te_fp8_gemm with
# constructed operands: v_mfma_*_f8f6f4 sums products in groups of 8 consecutive k;
# inside a group every product is truncated toward zero to a multiple of
# 2^(E - 13), E the exponent of the group's largest product (1 + 2^-13 is kept,
# 1 + 2^-14 and 1 - 2^-14 give 1, 16 + 2^-9 is kept, 64 + 2^-9 gives 64); group
# sums then accumulate in fp32.  The bound below uses a 12-bit window (a factor 2
# of margin over the measurement).
MFMA_GROUP = 8
MFMA_WINDOW_BITS = 12


def fp8_gemm_error_bound(a_vals, b_vals, scale, ref, out):
    """Per-element bound on |gpu - oracle| for D = scale * (A . B^T) [+ bias].

    a_vals [m, k], b_vals [n, k]: exact dequantized operand values (MX block scales
    already applied, per-tensor scales in `scale`); ref: the oracle's output."""
    A = np.abs(np.asarray(a_vals, dtype=np.float64))
    Bm = np.abs(np.asarray(b_vals, dtype=np.float64))
    m, k = A.shape
    n = Bm.shape[0]
    g = -(-k // MFMA_GROUP)
    pad = g * MFMA_GROUP - k
    if pad:
        A = np.pad(A, ((0, 0), (0, pad)))
        Bm = np.pad(Bm, ((0, 0), (0, pad)))
    amax = A.reshape(m, g, MFMA_GROUP).max(axis=2)
    bmax = Bm.reshape(n, g, MFMA_GROUP).max(axis=2)
    trunc = MFMA_GROUP * 2.0 ** -MFMA_WINDOW_BITS * (amax @ bmax.T)
    accum = (g + 4) * 2.0 ** -24 * (A @ Bm.T)
    e = abs(float(scale)) * (trunc + accum)
    mag = np.abs(np.asarray(ref, dtype=np.float64)) + e
    e = e + (2.0 ** -7 if out == "bf16" else 2.0 ** -22) * mag
    return e


def check_fp8_gemm(got, ref, a_vals, b_vals, scale, out):
    """Element-wise bound from the matrix-core arithmetic, and the normwise relative
    error within 1e-2 (bf16 out) / 1e-3 (fp32 out).  Returns (max excess ratio, normwise)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = fp8_gemm_error_bound(a_vals, b_vals, scale, ref, out)
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, diff / bound, np.where(diff > 0, np.inf, 0.0))
    ratio = float(np.max(r)) if diff.size else 0.0
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0
    worst = np.unravel_index(np.argmax(r), diff.shape) if diff.size else None
    assert ratio <= 1.0, f"outside the MFMA error bound at {worst}: |d-r|={diff[worst]:.4g} bound={bound[worst]:.4g}"
    assert nrm <= (1e-2 if out == "bf16" else 1e-3), f"normwise relative error {nrm:.3g}"
    return ratio, nrm
