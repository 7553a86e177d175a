"""Per-tensor scaling (current and delayed) and MXFP8 block quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * [FP8-intro] "FP8 Training について": one scaling factor per tensor (weights
    and activations each), because a single global scale as in FP16 loss
    scaling is not enough for FP8's narrow range; during training the ranges
    move every step, so the factor is refreshed every step.
  * [TE-summary] "主な機能": the scale is managed from an amax history.
  * [FP8-intro] "Transformer Engine の使い方": ``DelayedScaling(fp8_format=
    Format.HYBRID, amax_history_len=16, amax_compute_algo="max")``.
  * [FP8-intro] "Transformer Engine 統合済みライブラリの利用" (NeMo YAML):
    margin 0, update interval 1, ``amax_compute_algo`` is ``max`` or
    ``most_recent``.
  * [LP-opt] "autocast モードの使用と事前量子化の比較": delayed scaling relies
    on the amax history; current scaling is named beside it.
  * [TE-summary] "主な機能" / [TE-readme]: MXFP8 (block-scaled FP8).

Readings where the pages are silent:
  * scale = fp8_max / amax in fp32 (correctly rounded division), times 2^-margin;
    overflow -> FLT_MAX; amax == 0 or non-finite -> 1.0 (current) or keep the
    previous scale (delayed);
  * scale_inv = fl32(1 / scale);
  * cast: q = encode(fl32(x * scale)) -- an fp32 multiply, then the FP8 encode;
  * delayed: the cast at step t uses the scale computed after step t-1, writes
    amax_t into history slot 0; the update takes max (or slot 0) over the
    history, then rolls it (slot i <- slot i-1, slot 0 <- 0);
  * MXFP8 (OCP MX v1.0 reading): blocks of 32 consecutive elements along the
    GEMM's reduction axis; E8M0 shared exponent e = floor(log2 amax_block) - 8
    (8 = exponent of E4M3's largest power of two), clamped to [-127, 127],
    code e + 127; an all-zero block gets code 127, an infinite amax
    (log2 = +inf) code 254; elements are encode_E4M3(x * 2^-e) (saturating).

Parity: amax, scale, cast, delayed update and MXFP8 are pinned by closed forms,
brute force and invariants in tests/test_oracle_quantize.py.  The MXFP8
zero-block code and the clip-versus-round-up choice for the shared exponent are
readings of the OCP spec only (parity unpinned for those two choices).
"""

from __future__ import annotations

import numpy as np

from .formats import FP8Format, E4M3, encode

FLT_MAX = np.float32(np.finfo(np.float32).max)


def amax(x) -> np.float32:
    """max_i |x_i| of the tensor, as fp32 (exact: no arithmetic besides abs)."""
    x32 = np.asarray(x, dtype=np.float32)
    if x32.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x32)))


def _fp8_max32(fmt: FP8Format) -> np.float32:
    return np.float32(fmt.max)


def _apply_margin(s: np.float32, margin: int) -> np.float32:
    # 2^-margin is a power of two: the product is exact unless it underflows
    return np.float32(np.ldexp(np.float64(s), -int(margin)))


def current_scale(am, fmt: FP8Format, margin: int = 0) -> np.float32:
    """Current scaling: the scale comes from this tensor's own amax.

    [LP-opt] section "実モデルにおける結果の解釈" (FP8 CurrentScaling bullet)
    names the recipe; the formula is the reading stated in the module header.
    """
    am = np.float32(am)
    if not np.isfinite(am) or am == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore"):
        s = np.float32(_fp8_max32(fmt) / am)  # IEEE fp32 division (correctly rounded)
    if not np.isfinite(s):
        s = FLT_MAX
    return _apply_margin(s, margin)


def scale_inverse(s) -> np.float32:
    with np.errstate(over="ignore", divide="ignore"):
        return np.float32(np.float32(1.0) / np.float32(s))


def scaled_cast(x, scale, fmt: FP8Format) -> np.ndarray:
    """q_i = encode(fl32(x_i * scale)): fp32 multiply, then saturating RNE encode.

    [FP8-intro] "FP8 Training について": each tensor is scaled by its own factor
    and converted to FP8.
    """
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = x32 * np.float32(scale)  # numpy float32 multiply: IEEE, round to nearest even
    return encode(prod, fmt)


def cast_transpose(x, scale, fmt: FP8Format):
    """The scaled cast in the input's layout and its byte transpose.

    Not named on the pages; it follows from the TN GEMM layout: the Dgrad and
    Wgrad GEMMs of [LP-opt] "autocast モードの使用と事前量子化の比較" need W,
    X and dY with the other dimension contiguous.
    """
    row = scaled_cast(x, scale, fmt)
    return row, np.ascontiguousarray(row.T)


def delayed_update(hist, scale, fmt: FP8Format, algo: str = "max", margin: int = 0):
    """One scale update for one tensor of a delayed-scaling recipe.

    Takes the amax history (slot 0 = newest) and the previous scale; returns
    (new_hist, new_scale, new_scale_inv).  Order: reduce the history, compute
    the scale, then roll the history so slot 0 is free for the next step.
    [FP8-intro] "Transformer Engine の使い方" (amax_history_len, algo "max") and
    the NeMo keys ``fp8_amax_compute_algo: max # 'most_recent' or 'max'``.
    """
    hist = np.asarray(hist, dtype=np.float32).copy()
    if algo == "max":
        a = np.float32(np.max(hist))
    elif algo == "most_recent":
        a = np.float32(hist[0])
    else:
        raise ValueError(algo)
    if np.isfinite(a) and a > 0:
        with np.errstate(over="ignore"):
            s = np.float32(_fp8_max32(fmt) / a)
        if not np.isfinite(s):
            s = FLT_MAX
        s = _apply_margin(s, margin)
    else:
        s = np.float32(scale)
    new_hist = np.empty_like(hist)
    new_hist[1:] = hist[:-1]
    new_hist[0] = 0.0
    return new_hist, s, scale_inverse(s)


class DelayedScalingState:
    """Scaling state of one tensor under delayed scaling.

    Initial state: zero history, scale 1, scale_inv 1.  ``cast`` quantizes with
    the current scale and records amax into slot 0; ``update`` refreshes the
    scale from the history and rolls it (interval 1: after every step).
    """

    def __init__(self, fmt: FP8Format, history_len: int = 16, algo: str = "max", margin: int = 0):
        self.fmt = fmt
        self.hist = np.zeros(history_len, dtype=np.float32)
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.algo = algo
        self.margin = margin

    def cast(self, x):
        self.hist[0] = amax(x)
        return scaled_cast(x, self.scale, self.fmt), self.scale_inv

    def update(self):
        self.hist, self.scale, self.scale_inv = delayed_update(
            self.hist, self.scale, self.fmt, self.algo, self.margin)


def e8m0_to_float(code) -> np.ndarray:
    """E8M0 code -> 2^(code - 127) as float64 (code 255, NaN, is never produced)."""
    c = np.asarray(code, dtype=np.int64)
    return np.ldexp(1.0, (c - 127).astype(np.int32))


def _floor_log2(a64: np.ndarray) -> np.ndarray:
    _, e = np.frexp(a64)
    return e.astype(np.int64) - 1


def mxfp8_quantize(x, fmt: FP8Format = E4M3, block: int = 32):
    """MXFP8 quantization of each row of ``x`` in blocks of ``block`` along the row.

    Returns (codes uint8 [R, C], e8m0 uint8 [R, C/block]).  The column-wise copy
    used by the Dgrad/Wgrad GEMMs is ``mxfp8_quantize(x.T)``: an independent
    quantization with blocks along the other axis.
    """
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    if C % block:
        raise ValueError("row length must be a multiple of the block size")
    xb = x32.reshape(R, C // block, block).astype(np.float64)
    am = np.max(np.abs(xb), axis=2)
    # exponent of the element format's largest power of two (256 for E4M3, 2^15 for E5M2)
    emax_elem = int(np.floor(np.log2(fmt.max)))
    fin = np.isfinite(am)
    pos = (am > 0) & fin
    e = np.where(pos, _floor_log2(np.where(pos, am, 1.0)) - emax_elem, 0)
    e = np.where(np.isinf(am), 127, e)  # log2 of an infinite amax is +inf: the clamp's top
    e = np.clip(e, -127, 127)
    codes_e8m0 = (e + 127).astype(np.uint8)
    scaled = np.ldexp(xb, (-e)[:, :, None].astype(np.int32)).astype(np.float32)
    q = encode(scaled, fmt).reshape(R, C)
    return q, codes_e8m0


def mx_scales_panel(e8m0, panel: int = 256) -> np.ndarray:
    """E8M0 block scales [R, C/32] (row r, block b along the row) rearranged into the
    panel layout a GEMM reads a k stage at a time: rows in panels of 256; within a
    panel, for each group of four consecutive blocks g (128 elements), the 256 rows'
    dwords of that group are contiguous.  Byte of (r, b):
        4 * ((r // 256) * G + b // 4) * 256 + 4 * (r % 256) + b % 4,   G = C / 128.
    Returns uint8 [ceil(R / 256) * 256 * G * 4]; bytes of the padding rows of the last
    panel are 127 (they belong to no row).  Needs C % 128 == 0.

    Not on the pages: the layout only reorders the scales of the MX block rule (OCP MX
    v1.0 reading of [TE-summary] "主な機能" MXFP8), so that the four scale bytes of one
    row and 128-element stage are one dword and a stage's dwords of 256 rows are one
    contiguous kilobyte."""
    e = np.asarray(e8m0, dtype=np.uint8)
    R, nb = e.shape
    if nb % 4:
        raise ValueError("the panel layout needs a multiple of four blocks (128 elements) per row")
    G = nb // 4
    P = -(-R // panel)
    out = np.full(P * panel * G * 4, 127, np.uint8)
    for r in range(R):
        for b in range(nb):
            out[4 * ((r // panel) * G + b // 4) * panel + 4 * (r % panel) + b % 4] = e[r, b]
    return out


def mx_scales_from_panel(panel_bytes, rows: int, blocks: int, panel: int = 256) -> np.ndarray:
    """Inverse of mx_scales_panel: [rows, blocks] E8M0 from the panel layout."""
    p = np.asarray(panel_bytes, dtype=np.uint8)
    G = blocks // 4
    out = np.empty((rows, blocks), np.uint8)
    for r in range(rows):
        for b in range(blocks):
            out[r, b] = p[4 * ((r // panel) * G + b // 4) * panel + 4 * (r % panel) + b % 4]
    return out
