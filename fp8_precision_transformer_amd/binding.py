"""Thin Python binding of libte_mi355x.so: argument marshalling only.

Every call takes torch tensors that already live on the GPU, checks that they
are contiguous and on one device, passes their data pointers, sizes and dtype
codes to the C ABI (include/te_mi355x.h) together with the current HIP stream,
and raises ``TEError`` with the library's message on any non-OK status.  No
arithmetic of the method happens here; there is no fallback: if the library is
missing, loading fails loudly.

The library must bind to the same HIP runtime as PyTorch so that streams and
device pointers are shared.  PyTorch is imported first; the library's
dependency on ``libamdhip64.so.7`` is then satisfied by the copy already loaded.
"""

from __future__ import annotations

import ctypes
import os
import re
import threading

import torch  # noqa: F401  (loads PyTorch's HIP runtime before the library)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libte_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "te_mi355x.h")

# te_status
TE_OK, TE_ERR_NULL, TE_ERR_SHAPE, TE_ERR_DTYPE, TE_ERR_ALIGN, TE_ERR_UNSUPPORTED, TE_ERR_HIP, TE_ERR_ARG = range(8)
STATUS_NAMES = ["TE_OK", "TE_ERR_NULL", "TE_ERR_SHAPE", "TE_ERR_DTYPE", "TE_ERR_ALIGN",
                "TE_ERR_UNSUPPORTED", "TE_ERR_HIP", "TE_ERR_ARG"]
# te_dtype
TE_F32, TE_BF16, TE_E4M3, TE_E5M2, TE_E8M0, TE_E2M1 = range(6)
# te_scaling, te_amax_algo, te_granularity
TE_SCALE_DELAYED, TE_SCALE_CURRENT, TE_SCALE_CURRENT_FROM_AMAX = 0, 1, 2
TE_AMAX_MAX, TE_AMAX_MOST_RECENT = 0, 1
TE_GRAN_TENSOR, TE_GRAN_MX_BLOCK32, TE_GRAN_MX_BLOCK32_PANEL = 0, 1, 2
# te_mxfp4_quantize_recipe flags
TE_MX4_RHT, TE_MX4_SR, TE_MX4_2D = 1, 2, 4

FP8_CODES = {"E4M3": TE_E4M3, "E5M2": TE_E5M2, "E2M1": TE_E2M1}


class TEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()

_vp, _i64, _i32, _fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p

_SIGNATURES = {
    "te_amax_cast": [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "te_cast_transpose": [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "te_layernorm_fp8": [_vp, _i32, _i64, _i64, _vp, _vp, _i32, ctypes.c_float, _i32, _i32, _i32, _vp, _vp, _vp,
                         _vp, _vp, _vp, _vp, _vp],
    "te_cast_transpose_dbias": [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                _vp],
    "te_cast_transpose_dbias_noalloc": [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp],
    "te_scale_update": [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp],
    "te_fp8_gemm": [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _vp],
    "te_fp8_gemm_amax": [_vp, _i32, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                         _vp, _vp],
    "te_fp8_gemm_accumulate": [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp, _vp],
    "te_mxfp8_quantize": [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp],
    "te_mxfp8_quantize_dbias": [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp],
    "te_mxfp4_quantize": [_vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "te_mxfp8_quantize_panel": [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp],
    "te_fp8_gemm_splitk": [_vp, _i32, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _i32, _vp, _i64,
                           _vp],
    "te_mxfp4_quantize_recipe": [_vp, _i32, _i64, _i64, _i32, ctypes.c_uint32, ctypes.c_uint64, _vp, _vp, _vp, _vp,
                                 _vp],
    "te_mxfp4_quantize_panel": [_vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
}


def lib() -> ctypes.CDLL:
    """Load libte_mi355x.so (built by ``__graft_entry__.build()``); raises if missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                    "(there is no CPU or PyTorch fallback for this path)")
            L = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGNATURES.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = ctypes.c_int
            L.te_get_last_error.restype = ctypes.c_char_p
            L.te_get_last_error.argtypes = []
            L.te_version.restype = ctypes.c_char_p
            L.te_version.argtypes = []
            L.te_gemm_variant.restype = ctypes.c_char_p
            L.te_gemm_variant.argtypes = []
            L.te_cast_transpose_dbias_workspace_bytes.restype = ctypes.c_int64
            L.te_cast_transpose_dbias_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
            L.te_mxfp8_quantize_dbias_workspace_bytes.restype = ctypes.c_int64
            L.te_mxfp8_quantize_dbias_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
            L.te_mx_scale_panel_bytes.restype = ctypes.c_int64
            L.te_mx_scale_panel_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
            L.te_fp8_gemm_splitk_workspace_bytes.restype = ctypes.c_int64
            L.te_fp8_gemm_splitk_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
            L.te_amax_workspace_bytes.restype = ctypes.c_int64
            L.te_amax_workspace_bytes.argtypes = []
            L.te_cast_transpose_dbias_noalloc_max_bytes.restype = ctypes.c_int64
            L.te_cast_transpose_dbias_noalloc_max_bytes.argtypes = []
            _lib = L
    return _lib


def header_functions(path: str = HEADER):
    """Names of the functions include/te_mi355x.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(te_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != TE_OK:
        raise TEError(status, lib().te_get_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _hp_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TE_F32
    if t.dtype == torch.bfloat16:
        return TE_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _fp8_code(fmt) -> int:
    if isinstance(fmt, int):
        return fmt
    return FP8_CODES[str(fmt).upper()]


def _need(t: torch.Tensor, name: str, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _2d(x: torch.Tensor):
    if x.dim() == 2:
        return x.shape[0], x.shape[1]
    if x.dim() == 1:
        return 1, x.shape[0]
    return x.numel() // x.shape[-1], x.shape[-1]


def te_amax_workspace_bytes() -> int:
    return int(lib().te_amax_workspace_bytes())


def amax_workspace(device=None) -> torch.Tensor:
    """A new zeroed amax workspace (te_amax_workspace_bytes() bytes) on `device`, for the
    caller to keep and pass to the amax-producing calls.  Calls that may run at the
    same time need different workspaces."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    return torch.zeros(te_amax_workspace_bytes(), dtype=torch.uint8, device=dev)


def te_amax_cast(x, out_dtype, mode, margin, scale, scale_inv, amax, out=None, workspace=None, stream=None):
    """workspace: an amax workspace (amax_workspace()); None only for TE_SCALE_CURRENT_FROM_AMAX."""
    for n, t in (("x", x), ("scale", scale), ("scale_inv", scale_inv), ("amax", amax), ("out", out),
                 ("workspace", workspace)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_amax_cast(_ptr(x), _hp_code(x), rows, cols, _fp8_code(out_dtype), int(mode), int(margin),
                              _ptr(scale), _ptr(scale_inv), _ptr(amax), _ptr(out), _ptr(workspace),
                              _stream(stream)))


def te_cast_transpose(x, out_dtype, mode, margin, scale, scale_inv, amax, out_row=None, out_col=None,
                      workspace=None, stream=None):
    for n, t in (("x", x), ("scale", scale), ("scale_inv", scale_inv), ("amax", amax),
                 ("out_row", out_row), ("out_col", out_col), ("workspace", workspace)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_cast_transpose(_ptr(x), _hp_code(x), rows, cols, _fp8_code(out_dtype), int(mode),
                                   int(margin), _ptr(scale), _ptr(scale_inv), _ptr(amax), _ptr(out_row),
                                   _ptr(out_col), _ptr(workspace), _stream(stream)))


def te_mx_scale_panel_bytes(rows, cols) -> int:
    """Bytes of E8M0 scales in the panel layout for [rows, cols] (cols % 128 == 0)."""
    return int(lib().te_mx_scale_panel_bytes(int(rows), int(cols)))


def te_cast_transpose_dbias_workspace_bytes(rows, cols) -> int:
    return int(lib().te_cast_transpose_dbias_workspace_bytes(int(rows), int(cols)))


def dbias_workspace(rows, cols, device=None) -> torch.Tensor:
    """A new workspace for te_cast_transpose_dbias of [rows, cols] (its amax part zeroed)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    return torch.zeros(te_cast_transpose_dbias_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)


def te_cast_transpose_dbias(x, out_dtype, mode, margin, scale, scale_inv, amax, dbias, workspace,
                            out_row=None, out_col=None, stream=None):
    """te_cast_transpose plus dbias[c] = sum_r x[r, c] (fp32) from the same pass; workspace:
    a device tensor of at least te_cast_transpose_dbias_workspace_bytes(rows, cols) bytes whose
    first te_amax_workspace_bytes() bytes are an amax workspace (dbias_workspace())."""
    for n, t in (("x", x), ("scale", scale), ("scale_inv", scale_inv), ("amax", amax),
                 ("out_row", out_row), ("out_col", out_col), ("dbias", dbias), ("workspace", workspace)):
        _need(t, n)
    rows, cols = _2d(x)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().te_cast_transpose_dbias(_ptr(x), _hp_code(x), rows, cols, _fp8_code(out_dtype), int(mode),
                                         int(margin), _ptr(scale), _ptr(scale_inv), _ptr(amax), _ptr(out_row),
                                         _ptr(out_col), _ptr(dbias), _ptr(workspace), ws_bytes, _stream(stream)))


def te_cast_transpose_dbias_noalloc(x, out_dtype, mode, margin, scale, scale_inv, amax, dbias, out_row=None,
                                    out_col=None, stream=None):
    """te_cast_transpose_dbias with the library's static scratch instead of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    for n, t in (("x", x), ("scale", scale), ("scale_inv", scale_inv), ("amax", amax),
                 ("out_row", out_row), ("out_col", out_col), ("dbias", dbias)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_cast_transpose_dbias_noalloc(_ptr(x), _hp_code(x), rows, cols, _fp8_code(out_dtype), int(mode),
                                                 int(margin), _ptr(scale), _ptr(scale_inv), _ptr(amax),
                                                 _ptr(out_row), _ptr(out_col), _ptr(dbias), _stream(stream)))


def te_cast_transpose_dbias_noalloc_max_bytes() -> int:
    return int(lib().te_cast_transpose_dbias_noalloc_max_bytes())


def te_layernorm_fp8(x, gamma, beta, eps, out_dtype, mode, margin, scale, scale_inv, amax, out, mu=None,
                     rsigma=None, workspace=None, stream=None):
    """LayerNorm of x over its last axis, written as FP8 codes into out (see the header);
    workspace: an amax workspace (amax_workspace())."""
    for n, t in (("x", x), ("gamma", gamma), ("beta", beta), ("scale", scale), ("scale_inv", scale_inv),
                 ("amax", amax), ("out", out), ("mu", mu), ("rsigma", rsigma), ("workspace", workspace)):
        _need(t, n)
    if gamma.dtype != beta.dtype:
        raise ValueError("gamma and beta must share a dtype")
    rows, cols = _2d(x)
    _check(lib().te_layernorm_fp8(_ptr(x), _hp_code(x), rows, cols, _ptr(gamma), _ptr(beta), _hp_code(gamma),
                                  float(eps), _fp8_code(out_dtype), int(mode), int(margin), _ptr(scale),
                                  _ptr(scale_inv), _ptr(amax), _ptr(out), _ptr(mu), _ptr(rsigma), _ptr(workspace),
                                  _stream(stream)))


def te_scale_update(amax_history, scale, scale_inv, fp8_dtype, algo=TE_AMAX_MAX, margin=0, stream=None):
    for n, t in (("amax_history", amax_history), ("scale", scale), ("scale_inv", scale_inv)):
        _need(t, n, torch.float32)
    n_t, hist_len = (amax_history.shape[0], amax_history.shape[1]) if amax_history.dim() == 2 else (1, amax_history.shape[0])
    _check(lib().te_scale_update(_ptr(amax_history), _ptr(scale), _ptr(scale_inv), n_t, hist_len,
                                 _fp8_code(fp8_dtype), int(algo), int(margin), _stream(stream)))


def te_fp8_gemm(a, a_dtype, a_scale, b, b_dtype, b_scale, d, bias=None, gran=TE_GRAN_TENSOR, stream=None,
                accumulate=False):
    """D[m, n] = A[m, k] . B[n, k]^T.  a, b: uint8 FP8 codes (or bf16 tensors with
    a_dtype = b_dtype = "BF16", or packed MXFP4 codes [m, k/2], [n, k/2] with
    a_dtype = b_dtype = "E2M1"); a_scale/b_scale: fp32 [1] scale_inv or uint8 E8M0.
    accumulate=True (fp32 d only) adds the result into d (te_fp8_gemm_accumulate)."""
    for n, t in (("a", a), ("b", b), ("d", d), ("bias", bias), ("a_scale", a_scale), ("b_scale", b_scale)):
        _need(t, n)
    ad = TE_BF16 if str(a_dtype).upper() == "BF16" else _fp8_code(a_dtype)
    bd = TE_BF16 if str(b_dtype).upper() == "BF16" else _fp8_code(b_dtype)
    m, kb = a.shape
    n = b.shape[0]
    if b.shape[1] != kb:
        raise ValueError(f"k mismatch: a {tuple(a.shape)} b {tuple(b.shape)}")
    k = 2 * kb if ad == TE_E2M1 else kb  # E2M1: two elements per byte
    if tuple(d.shape) != (m, n):
        raise ValueError(f"d must be [{m}, {n}]")
    dd = _hp_code(d)
    bias_code = _hp_code(bias) if bias is not None else TE_F32
    if accumulate:
        if dd != TE_F32:
            raise ValueError("accumulate needs an fp32 d")
        _check(lib().te_fp8_gemm_accumulate(_ptr(a), ad, _ptr(a_scale), _ptr(b), bd, _ptr(b_scale), int(gran), m,
                                            n, k, _ptr(bias), bias_code, _ptr(d), _stream(stream)))
        return
    _check(lib().te_fp8_gemm(_ptr(a), ad, _ptr(a_scale), _ptr(b), bd, _ptr(b_scale), int(gran), m, n, k,
                             _ptr(bias), bias_code, _ptr(d), dd, _stream(stream)))


def te_fp8_gemm_amax(a, a_dtype, a_scale, b, b_dtype, b_scale, d, amax, workspace, bias=None, d_scale=None,
                     d_scale_inv=None, stream=None):
    """te_fp8_gemm (per-tensor FP8 or BF16) that also writes amax = max |D| of the stored bf16
    or fp32 output d; workspace: an amax workspace.  FP8 output: te_fp8_gemm_amax_fp8."""
    for n_, t in (("a", a), ("b", b), ("d", d), ("bias", bias), ("a_scale", a_scale), ("b_scale", b_scale),
                  ("amax", amax), ("workspace", workspace)):
        _need(t, n_)
    ad = TE_BF16 if str(a_dtype).upper() == "BF16" else _fp8_code(a_dtype)
    bd = TE_BF16 if str(b_dtype).upper() == "BF16" else _fp8_code(b_dtype)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)} b {tuple(b.shape)} d {tuple(d.shape)}")
    bias_code = _hp_code(bias) if bias is not None else TE_F32
    _check(lib().te_fp8_gemm_amax(_ptr(a), ad, _ptr(a_scale), _ptr(b), bd, _ptr(b_scale), m, n, k, _ptr(bias),
                                  bias_code, _ptr(d), _hp_code(d), None, None, _ptr(amax), _ptr(workspace),
                                  _stream(stream)))


def te_fp8_gemm_amax_fp8(a, a_dtype, a_scale, b, b_dtype, b_scale, d, d_dtype, d_scale, d_scale_inv, amax,
                         workspace, bias=None, stream=None):
    """te_fp8_gemm_amax writing D [m, n] as FP8 codes (uint8) of d_dtype ("E4M3"/"E5M2")
    with the scale d_scale; d_scale_inv written; amax of the fp32 results before the cast."""
    for n_, t in (("a", a), ("b", b), ("d", d), ("bias", bias), ("a_scale", a_scale), ("b_scale", b_scale),
                  ("d_scale", d_scale), ("d_scale_inv", d_scale_inv), ("amax", amax), ("workspace", workspace)):
        _need(t, n_)
    ad = TE_BF16 if str(a_dtype).upper() == "BF16" else _fp8_code(a_dtype)
    bd = TE_BF16 if str(b_dtype).upper() == "BF16" else _fp8_code(b_dtype)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n) or d.dtype != torch.uint8:
        raise ValueError(f"shape mismatch: a {tuple(a.shape)} b {tuple(b.shape)} d {tuple(d.shape)} {d.dtype}")
    bias_code = _hp_code(bias) if bias is not None else TE_F32
    _check(lib().te_fp8_gemm_amax(_ptr(a), ad, _ptr(a_scale), _ptr(b), bd, _ptr(b_scale), m, n, k, _ptr(bias),
                                  bias_code, _ptr(d), _fp8_code(d_dtype), _ptr(d_scale), _ptr(d_scale_inv),
                                  _ptr(amax), _ptr(workspace), _stream(stream)))


def te_fp8_gemm_splitk_workspace_bytes(m, n, splits) -> int:
    return int(lib().te_fp8_gemm_splitk_workspace_bytes(int(m), int(n), int(splits)))


def te_fp8_gemm_splitk(a, a_dtype, a_scale, b, b_dtype, b_scale, d, splits, workspace, bias=None, stream=None):
    """te_fp8_gemm (per-tensor FP8 or BF16) with k split `splits` ways; workspace: a device
    tensor of at least te_fp8_gemm_splitk_workspace_bytes(m, n, splits) bytes."""
    for n_, t in (("a", a), ("b", b), ("d", d), ("bias", bias), ("a_scale", a_scale), ("b_scale", b_scale),
                  ("workspace", workspace)):
        _need(t, n_)
    ad = TE_BF16 if str(a_dtype).upper() == "BF16" else _fp8_code(a_dtype)
    bd = TE_BF16 if str(b_dtype).upper() == "BF16" else _fp8_code(b_dtype)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)} b {tuple(b.shape)} d {tuple(d.shape)}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    bias_code = _hp_code(bias) if bias is not None else TE_F32
    _check(lib().te_fp8_gemm_splitk(_ptr(a), ad, _ptr(a_scale), _ptr(b), bd, _ptr(b_scale), m, n, k, _ptr(bias),
                                    bias_code, _ptr(d), _hp_code(d), int(splits), _ptr(workspace), ws_bytes,
                                    _stream(stream)))


def te_mxfp8_quantize(x, elem_dtype, out_row=None, scale_row=None, out_col=None, scale_col=None, stream=None):
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_mxfp8_quantize(_ptr(x), _hp_code(x), rows, cols, _fp8_code(elem_dtype), _ptr(out_row),
                                   _ptr(scale_row), _ptr(out_col), _ptr(scale_col), _stream(stream)))


def te_mxfp8_quantize_dbias_workspace_bytes(rows, cols) -> int:
    return int(lib().te_mxfp8_quantize_dbias_workspace_bytes(int(rows), int(cols)))


def mx_dbias_workspace(rows, cols, device=None) -> torch.Tensor:
    """A new workspace for te_mxfp8_quantize_dbias of [rows, cols] (no initial contents needed)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    return torch.empty(max(te_mxfp8_quantize_dbias_workspace_bytes(rows, cols), 16), dtype=torch.uint8, device=dev)


def te_mxfp8_quantize_dbias(x, elem_dtype, dbias, workspace, out_row=None, scale_row=None, out_col=None,
                            scale_col=None, stream=None):
    """te_mxfp8_quantize plus dbias[c] = sum_r x[r, c] (fp32) from the same pass."""
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col), ("dbias", dbias), ("workspace", workspace)):
        _need(t, n)
    rows, cols = _2d(x)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().te_mxfp8_quantize_dbias(_ptr(x), _hp_code(x), rows, cols, _fp8_code(elem_dtype), _ptr(out_row),
                                         _ptr(scale_row), _ptr(out_col), _ptr(scale_col), _ptr(dbias),
                                         _ptr(workspace), ws_bytes, _stream(stream)))


def te_mxfp4_quantize(x, out_row=None, scale_row=None, out_col=None, scale_col=None, stream=None):
    """MXFP4 of x: out_row uint8 [rows, cols/2] (two codes per byte) with scale_row
    [rows, cols/32]; out_col uint8 [cols, rows/2] with scale_col [cols, rows/32]."""
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_mxfp4_quantize(_ptr(x), _hp_code(x), rows, cols, _ptr(out_row), _ptr(scale_row),
                                   _ptr(out_col), _ptr(scale_col), _stream(stream)))


def te_mxfp8_quantize_panel(x, elem_dtype, out_row=None, scale_row=None, out_col=None, scale_col=None,
                            stream=None):
    """te_mxfp8_quantize with the scales in the panel layout: scale_row uint8
    [te_mx_scale_panel_bytes(rows, cols)], scale_col [te_mx_scale_panel_bytes(cols, rows)]."""
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_mxfp8_quantize_panel(_ptr(x), _hp_code(x), rows, cols, _fp8_code(elem_dtype), _ptr(out_row),
                                         _ptr(scale_row), _ptr(out_col), _ptr(scale_col), _stream(stream)))


def te_mxfp4_quantize_panel(x, out_row=None, scale_row=None, out_col=None, scale_col=None, stream=None):
    """te_mxfp4_quantize with the scales in the panel layout (see te_mxfp8_quantize_panel)."""
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_mxfp4_quantize_panel(_ptr(x), _hp_code(x), rows, cols, _ptr(out_row), _ptr(scale_row),
                                         _ptr(out_col), _ptr(scale_col), _stream(stream)))


def te_mxfp4_quantize_recipe(x, flags, out_row=None, scale_row=None, out_col=None, scale_col=None, sign_mask=0,
                             seed=0, stream=None):
    """MXFP4 with the FP4 recipe steps (TE_MX4_RHT / TE_MX4_SR / TE_MX4_2D), panel-layout scales."""
    for n, t in (("x", x), ("out_row", out_row), ("scale_row", scale_row), ("out_col", out_col),
                 ("scale_col", scale_col)):
        _need(t, n)
    rows, cols = _2d(x)
    _check(lib().te_mxfp4_quantize_recipe(_ptr(x), _hp_code(x), rows, cols, int(flags), int(sign_mask) & 0xFFFFFFFF,
                                          int(seed) & ((1 << 64) - 1), _ptr(out_row), _ptr(scale_row), _ptr(out_col),
                                          _ptr(scale_col), _stream(stream)))


def version() -> str:
    return lib().te_version().decode()


def te_gemm_variant() -> str:
    """Kernel variant of the last te_fp8_gemm on this thread."""
    return lib().te_gemm_variant().decode()
