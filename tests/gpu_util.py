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


_WS = []


def amax_ws() -> torch.Tensor:
    """A shared amax workspace for calls on the default stream (created on first use)."""
    from fp8_precision_transformer_amd import binding as B
    if not _WS:
        _WS.append(B.amax_workspace(torch.device(DEV)))
    return _WS[0]


def new_ws() -> torch.Tensor:
    """A fresh zeroed amax workspace (for calls on another stream)."""
    from fp8_precision_transformer_amd import binding as B
    return B.amax_workspace(torch.device(DEV))


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


# The GEMM acceptance check (the matrix-core error model and the reported maximum
# relative error) lives in mfma_model.py.
from mfma_model import check_fp8_gemm, gemm_error_bound  # noqa: E402,F401
