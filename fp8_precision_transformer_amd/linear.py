"""``Linear`` and ``fp8_autocast``: the thin PyTorch layer over the C ABI.

[FP8-intro] "Transformer Engine の使い方": ``te.Linear(768, 768, bias=True)``
under ``te.fp8_autocast(enabled=True, fp8_recipe=...)``; the module keeps the
scaling factors and amax history of its tensors.  [FP8-intro] "fp8_autocast
の使用": only the forward pass is wrapped; backward runs outside it and uses
E5M2 for gradients under HYBRID.  [FP8-intro] "HuggingFace BERT を例にした
Transformer Engine の適用": both weight dimensions must be multiples of 16.

Every tensor operation of the FP8 path is a call into libte_mi355x.so: casts,
cast-transposes, scale updates and the Fprop/Dgrad/Wgrad GEMMs.  Outside
``fp8_autocast`` the layer computes in bf16 with the library's BF16 GEMM.

Scaling state per module (delayed scaling): ``amax_history`` [3, L], ``scale``
[3], ``scale_inv`` [3] fp32 device tensors; index 0 = input, 1 = weight,
2 = output gradient.  The forward-pass entries are updated when the autocast
region exits, the gradient entry at the end of backward (update interval 1).

The bias gradient comes from the pass that casts dY (te_cast_transpose_dbias).
With the MXFP8 recipe the forward pass also keeps the column-wise MX copies of x
and W (blocks along the token and output axes), which Wgrad and Dgrad take as
their k-contiguous operands; that needs a token count that is a multiple of 32.
"""

from __future__ import annotations

import contextlib
import threading

import torch

from . import binding as B
from .recipe import DelayedScaling, Float8CurrentScaling, MXFP8BlockScaling

_tls = threading.local()


class _AutocastState:
    def __init__(self, enabled, recipe):
        self.enabled = enabled
        self.recipe = recipe
        self.modules = []


def _current():
    return getattr(_tls, "state", None)


@contextlib.contextmanager
def fp8_autocast(enabled: bool = True, fp8_recipe=None):
    """Run the enclosed forward passes of ``Linear`` modules in FP8."""
    st = _AutocastState(enabled, fp8_recipe if fp8_recipe is not None else DelayedScaling())
    prev = _current()
    _tls.state = st
    try:
        yield
    finally:
        _tls.state = prev
        if enabled and isinstance(st.recipe, DelayedScaling):
            seen = set()
            for m in st.modules:
                if id(m) not in seen:
                    seen.add(id(m))
                    m._update_scales(slice(0, 2), st.recipe.fp8_format.forward_dtype(), st.recipe)


autocast = fp8_autocast


def _f8(n, dev):
    return torch.empty(n, dtype=torch.uint8, device=dev)


class _FP8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, weight, bias, module, recipe, need_grad):
        dev = x2.device
        M, K = x2.shape
        N = weight.shape[0]
        fwd = recipe.fp8_format.forward_dtype()
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ctx.module, ctx.recipe = module, recipe
        ctx.has_bias = bias is not None
        ctx.w_dtype = weight.dtype
        ctx.x_dtype = x2.dtype
        if isinstance(recipe, MXFP8BlockScaling):
            # row-wise copies for Fprop; with a backward, also the column-wise copies
            # (MX of x^T and W^T, blocks along M and N) for Wgrad and Dgrad
            if need_grad and M % 32:
                raise ValueError("MXFP8 backward needs a token count that is a multiple of 32")
            xq, xs = _f8((M, K), dev), _f8((M, K // 32), dev)
            wq, ws = _f8((N, K), dev), _f8((N, K // 32), dev)
            xqT = _f8((K, M), dev) if need_grad else None
            xsT = _f8((K, M // 32), dev) if need_grad else None
            wqT = _f8((K, N), dev) if need_grad else None
            wsT = _f8((K, N // 32), dev) if need_grad else None
            B.te_mxfp8_quantize(x2, fwd, xq, xs, xqT, xsT)
            B.te_mxfp8_quantize(weight, fwd, wq, ws, wqT, wsT)
            B.te_fp8_gemm(xq, fwd, xs, wq, fwd, ws, y, bias=bias, gran=B.TE_GRAN_MX_BLOCK32)
            if module.keep_fp8_tensors:
                module.last_fp8 = {"xq": xq, "xs": xs, "wq": wq, "ws": ws, "xqT": xqT, "xsT": xsT,
                                   "wqT": wqT, "wsT": wsT}
            ctx.save_for_backward(xqT, xsT, wqT, wsT)
            return y
        st = module._state(recipe)
        mode = B.TE_SCALE_CURRENT if isinstance(recipe, Float8CurrentScaling) else B.TE_SCALE_DELAYED
        margin = recipe.margin
        xq = _f8((M, K), dev)
        xqT = _f8((K, M), dev) if need_grad else None
        wq = _f8((N, K), dev)
        wqT = _f8((K, N), dev) if need_grad else None
        h, s, si = st["amax_history"], st["scale"], st["scale_inv"]
        B.te_cast_transpose(x2, fwd, mode, margin, s[0:1], si[0:1], h[0, 0:1], xq, xqT)
        B.te_cast_transpose(weight, fwd, mode, margin, s[1:2], si[1:2], h[1, 0:1], wq, wqT)
        B.te_fp8_gemm(xq, fwd, si[0:1], wq, fwd, si[1:2], y, bias=bias)
        if module.keep_fp8_tensors:
            module.last_fp8 = {"xq": xq, "wq": wq, "xqT": xqT, "wqT": wqT}
        ctx.mode = mode
        ctx.save_for_backward(xqT, wqT)
        return y

    @staticmethod
    def backward(ctx, dy):
        module, recipe = ctx.module, ctx.recipe
        bwd = recipe.fp8_format.backward_dtype()
        fwd = recipe.fp8_format.forward_dtype()
        dy = dy.contiguous()
        M, N = dy.shape
        dev = dy.device
        dx = dw = db = None
        if isinstance(recipe, MXFP8BlockScaling):
            xqT, xsT, wqT, wsT = ctx.saved_tensors
            K = xqT.shape[0]
            # dY row-wise (blocks along N, the k of Dgrad) and column-wise (blocks along
            # M, the k of Wgrad)
            dyq, dys = _f8((M, N), dev), _f8((M, N // 32), dev)
            dyqT, dysT = _f8((N, M), dev), _f8((N, M // 32), dev)
            if ctx.has_bias:
                db = _column_sums(dy, dyq)  # its codes are overwritten just below
            B.te_mxfp8_quantize(dy, bwd, dyq, dys, dyqT, dysT)
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            B.te_fp8_gemm(dyq, bwd, dys, wqT, fwd, wsT, dx, gran=B.TE_GRAN_MX_BLOCK32)      # Dgrad
            dw = torch.empty((N, K), dtype=torch.float32, device=dev)
            B.te_fp8_gemm(dyqT, bwd, dysT, xqT, fwd, xsT, dw, gran=B.TE_GRAN_MX_BLOCK32)    # Wgrad
            return dx.to(ctx.x_dtype), dw.to(ctx.w_dtype), db, None, None, None
        xqT, wqT = ctx.saved_tensors
        st = module._state(recipe)
        K = xqT.shape[0]
        h, s, si = st["amax_history"], st["scale"], st["scale_inv"]
        dyq, dyqT = _f8((M, N), dev), _f8((N, M), dev)
        if ctx.has_bias:  # bias gradient from the same pass over dY
            db = torch.empty(N, dtype=torch.float32, device=dev)
            ws = _f8(max(B.te_cast_transpose_dbias_workspace_bytes(M, N), 4), dev)
            B.te_cast_transpose_dbias(dy, bwd, ctx.mode, recipe.margin, s[2:3], si[2:3], h[2, 0:1], db, ws,
                                      dyq, dyqT)
        else:
            B.te_cast_transpose(dy, bwd, ctx.mode, recipe.margin, s[2:3], si[2:3], h[2, 0:1], dyq, dyqT)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        B.te_fp8_gemm(dyq, bwd, si[2:3], wqT, fwd, si[1:2], dx)              # Dgrad
        dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        B.te_fp8_gemm(dyqT, bwd, si[2:3], xqT, fwd, si[0:1], dw)             # Wgrad
        if isinstance(recipe, DelayedScaling):
            module._update_scales(slice(2, 3), bwd, recipe)
        return dx.to(ctx.x_dtype), dw.to(ctx.w_dtype), db, None, None, None


def _column_sums(dy, codes):
    """db[c] = sum_r dY[r, c] in fp32 by the library's dbias pass; the unit-scale E4M3
    codes it also writes go to `codes` [M, N] and are not used (MXFP8 quantizes dY
    itself)."""
    M, N = dy.shape
    dev = dy.device
    one = torch.ones(1, dtype=torch.float32, device=dev)
    si, am = torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
    db = torch.empty(N, dtype=torch.float32, device=dev)
    ws = _f8(max(B.te_cast_transpose_dbias_workspace_bytes(M, N), 4), dev)
    B.te_cast_transpose_dbias(dy, "E4M3", B.TE_SCALE_DELAYED, 0, one, si, am, db, ws, codes, None)
    return db


class Linear(torch.nn.Module):
    """y = x W^T + b with FP8 GEMMs inside ``fp8_autocast``."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 params_dtype: torch.dtype = torch.float32, device="cuda"):
        super().__init__()
        if in_features % 16 or out_features % 16:
            raise ValueError("in_features and out_features must be multiples of 16")
        self.in_features, self.out_features = in_features, out_features
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, dtype=params_dtype, device=device))
        self.bias = torch.nn.Parameter(torch.zeros(out_features, dtype=params_dtype, device=device)) if bias else None
        with torch.no_grad():
            self.weight.normal_(0.0, 0.02)
        self._fp8 = None
        self.keep_fp8_tensors = False  # debugging/tests: keep the last FP8 operands in last_fp8
        self.last_fp8 = None

    def _state(self, recipe):
        L = recipe.amax_history_len if isinstance(recipe, DelayedScaling) else 1
        if self._fp8 is None or self._fp8["amax_history"].shape[1] != L:
            dev = self.weight.device
            self._fp8 = {
                "amax_history": torch.zeros((3, L), dtype=torch.float32, device=dev),
                "scale": torch.ones(3, dtype=torch.float32, device=dev),
                "scale_inv": torch.ones(3, dtype=torch.float32, device=dev),
            }
        return self._fp8

    def fp8_state_dict(self):
        """The scaling state as plain tensors (checkpointable with torch.save)."""
        return {k: v.clone() for k, v in (self._fp8 or {}).items()}

    def load_fp8_state_dict(self, sd):
        self._fp8 = {k: v.clone().to(self.weight.device) for k, v in sd.items()}

    def _update_scales(self, idx: slice, fmt: str, recipe: DelayedScaling):
        st = self._fp8
        algo = B.TE_AMAX_MAX if recipe.amax_compute_algo == "max" else B.TE_AMAX_MOST_RECENT
        B.te_scale_update(st["amax_history"][idx], st["scale"][idx], st["scale_inv"][idx], fmt, algo, recipe.margin)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        st = _current()
        bias = self.bias
        if st is not None and st.enabled:
            if isinstance(st.recipe, DelayedScaling):
                st.modules.append(self)
            need_grad = torch.is_grad_enabled() and (x2.requires_grad or self.weight.requires_grad)
            y = _FP8LinearFn.apply(x2, self.weight, bias, self, st.recipe, need_grad)
        else:
            xb = x2.to(torch.bfloat16).contiguous()
            wb = self.weight.to(torch.bfloat16).contiguous()
            y = torch.empty((x2.shape[0], self.out_features), dtype=torch.bfloat16, device=x.device)
            B.te_fp8_gemm(xb, "BF16", None, wb, "BF16", None, y, bias=bias)
        return y.reshape(*lead, self.out_features)
