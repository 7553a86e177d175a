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

Scaling state (delayed scaling) lives in a pool per (device, history length,
gradient format): the input and weight of every module are rows of one amax
history [T, L] of the forward format (E4M3), the output gradients rows of one
history of the backward format, so ``fp8_autocast``'s exit updates each format
group with one ``te_scale_update`` launch ([FP8-intro] "Transformer Engine の使い
方": the amax history and scale of each FP8 tensor).  The forward-format group is
updated at every exit; the gradient group at the first exit after a backward pass
recorded gradient amaxes (update interval 1 for both).  The backward uses the
scale_inv values the forward casts used, saved at the forward (the exit's update
rewrites the pool before backward runs).

The bias gradient comes from the pass that casts dY (te_cast_transpose_dbias).
With the MXFP8 recipe the forward pass also keeps the column-wise MX copies of x
and W (blocks along the token and output axes), which Wgrad and Dgrad take as
their k-contiguous operands; that needs a token count that is a multiple of 32.

Amax workspaces (te_amax_workspace_bytes(), zeroed once) are kept per (device,
stream) in this module: calls on one stream run one after another and share one.
"""

from __future__ import annotations

import contextlib
import threading

import torch

from . import binding as B
from .recipe import DelayedScaling, Float8CurrentScaling, MXFP8BlockScaling

_tls = threading.local()
_ws_lock = threading.Lock()
_workspaces = {}  # (device index, stream handle) -> amax workspace


def _amax_workspace(dev: torch.device) -> torch.Tensor:
    """The amax workspace of (device, current stream), created zeroed on first use; not
    during stream capture (the zeroing would be captured, not run)."""
    stream = torch.cuda.current_stream(dev)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), stream.cuda_stream)
    with _ws_lock:
        ws = _workspaces.get(key)
        if ws is None:
            if torch.cuda.is_current_stream_capturing():
                raise RuntimeError("the first FP8 Linear call on a stream allocates its amax workspace; "
                                   "run one step eagerly before capturing")
            ws = B.amax_workspace(dev)
            _workspaces[key] = ws
    return ws


class _Group:
    """Delayed-scaling state of the tensors of one FP8 format: history [T, L] (slot 0
    newest), scale [T], scale_inv [T]; rows are appended as modules register."""

    def __init__(self, dev, L, fmt):
        self.fmt = fmt
        self.hist = torch.zeros((0, L), dtype=torch.float32, device=dev)
        self.scale = torch.ones(0, dtype=torch.float32, device=dev)
        self.scale_inv = torch.ones(0, dtype=torch.float32, device=dev)

    def add(self, n: int) -> int:
        i = self.hist.shape[0]
        dev, L = self.hist.device, self.hist.shape[1]
        self.hist = torch.cat([self.hist, torch.zeros((n, L), dtype=torch.float32, device=dev)])
        self.scale = torch.cat([self.scale, torch.ones(n, dtype=torch.float32, device=dev)])
        self.scale_inv = torch.cat([self.scale_inv, torch.ones(n, dtype=torch.float32, device=dev)])
        return i

    def update(self, recipe: DelayedScaling):
        if self.hist.shape[0] == 0:
            return
        algo = B.TE_AMAX_MAX if recipe.amax_compute_algo == "max" else B.TE_AMAX_MOST_RECENT
        B.te_scale_update(self.hist, self.scale, self.scale_inv, self.fmt, algo, recipe.margin)


class _ScalingPool:
    """The forward group (inputs and weights) and the gradient group of every module that
    runs delayed scaling on one device with one history length and gradient format."""

    def __init__(self, dev, L, bwd_fmt):
        self.fwd = _Group(dev, L, "E4M3")
        self.bwd = _Group(dev, L, bwd_fmt)
        self.bwd_pending = False  # a backward recorded gradient amaxes since the last update


_pools = {}


def _pool(dev: torch.device, recipe: DelayedScaling) -> _ScalingPool:
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, recipe.amax_history_len, recipe.fp8_format.backward_dtype())
    p = _pools.get(key)
    if p is None:
        p = _pools[key] = _ScalingPool(torch.device("cuda", idx), recipe.amax_history_len,
                                       recipe.fp8_format.backward_dtype())
    return p


class _AutocastState:
    def __init__(self, enabled, recipe):
        self.enabled = enabled
        self.recipe = recipe
        self.pools = {}  # id -> pool of the delayed-scaling modules run in this region


def _current():
    return getattr(_tls, "state", None)


@contextlib.contextmanager
def fp8_autocast(enabled: bool = True, fp8_recipe=None):
    """Run the enclosed forward passes of ``Linear`` modules in FP8.  With delayed
    scaling, the exit updates the scaling state: one te_scale_update per format group."""
    st = _AutocastState(enabled, fp8_recipe if fp8_recipe is not None else DelayedScaling())
    prev = _current()
    _tls.state = st
    try:
        yield
    finally:
        _tls.state = prev
        if enabled and isinstance(st.recipe, DelayedScaling):
            for pool in st.pools.values():
                pool.fwd.update(st.recipe)
                if pool.bwd_pending:
                    pool.bwd.update(st.recipe)
                    pool.bwd_pending = False


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
        mode = B.TE_SCALE_CURRENT if isinstance(recipe, Float8CurrentScaling) else B.TE_SCALE_DELAYED
        margin = recipe.margin
        xq = _f8((M, K), dev)
        xqT = _f8((K, M), dev) if need_grad else None
        wq = _f8((N, K), dev)
        wqT = _f8((K, N), dev) if need_grad else None
        (sx, sxi, ax), (sw, swi, aw), _ = module._slots(recipe)
        ws = _amax_workspace(dev)
        B.te_cast_transpose(x2, fwd, mode, margin, sx, sxi, ax, xq, xqT, workspace=ws)
        B.te_cast_transpose(weight, fwd, mode, margin, sw, swi, aw, wq, wqT, workspace=ws)
        B.te_fp8_gemm(xq, fwd, sxi, wq, fwd, swi, y, bias=bias)
        if module.keep_fp8_tensors:
            module.last_fp8 = {"xq": xq, "wq": wq, "xqT": xqT, "wqT": wqT}
        ctx.mode = mode
        # the scale_inv values these casts used (device copies, in stream order): with
        # delayed scaling the autocast exit rewrites the pool's before backward runs
        ctx.save_for_backward(xqT, wqT, torch.cat([sxi, swi]) if need_grad else None)
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
            if ctx.has_bias:  # bias gradient from the same pass over dY
                db = torch.empty(N, dtype=torch.float32, device=dev)
                B.te_mxfp8_quantize_dbias(dy, bwd, db, B.mx_dbias_workspace(M, N, dev), dyq, dys, dyqT, dysT)
            else:
                B.te_mxfp8_quantize(dy, bwd, dyq, dys, dyqT, dysT)
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            B.te_fp8_gemm(dyq, bwd, dys, wqT, fwd, wsT, dx, gran=B.TE_GRAN_MX_BLOCK32)      # Dgrad
            dw = torch.empty((N, K), dtype=torch.float32, device=dev)
            B.te_fp8_gemm(dyqT, bwd, dysT, xqT, fwd, xsT, dw, gran=B.TE_GRAN_MX_BLOCK32)    # Wgrad
            return dx.to(ctx.x_dtype), dw.to(ctx.w_dtype), db, None, None, None
        xqT, wqT, si_fwd = ctx.saved_tensors
        K = xqT.shape[0]
        _, _, (sg, sgi, ag) = module._slots(recipe)
        dyq, dyqT = _f8((M, N), dev), _f8((N, M), dev)
        if ctx.has_bias:  # bias gradient from the same pass over dY
            db = torch.empty(N, dtype=torch.float32, device=dev)
            ws = B.dbias_workspace(M, N, dev)
            B.te_cast_transpose_dbias(dy, bwd, ctx.mode, recipe.margin, sg, sgi, ag, db, ws, dyq, dyqT)
        else:
            B.te_cast_transpose(dy, bwd, ctx.mode, recipe.margin, sg, sgi, ag, dyq, dyqT,
                                workspace=_amax_workspace(dev))
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        B.te_fp8_gemm(dyq, bwd, sgi, wqT, fwd, si_fwd[1:2], dx)              # Dgrad
        dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        B.te_fp8_gemm(dyqT, bwd, sgi, xqT, fwd, si_fwd[0:1], dw)             # Wgrad
        if isinstance(recipe, DelayedScaling):
            module._fp8[_recipe_key(recipe)]["pool"].bwd_pending = True
        return dx.to(ctx.x_dtype), dw.to(ctx.w_dtype), db, None, None, None


def _recipe_key(recipe):
    if isinstance(recipe, DelayedScaling):
        return ("delayed", recipe.amax_history_len, recipe.fp8_format.backward_dtype())
    return ("current",)


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

    def _slots(self, recipe):
        """(scale, scale_inv, amax) views of the input, weight and output gradient: rows of
        the delayed-scaling pool (registered on first use), or this module's own scalars
        for current scaling."""
        key = _recipe_key(recipe)
        if self._fp8 is None:
            self._fp8 = {}
        st = self._fp8.get(key)
        dev = self.weight.device
        if st is None:
            if key[0] == "delayed":
                pool = _pool(dev, recipe)
                st = {"pool": pool, "fwd": pool.fwd.add(2), "bwd": pool.bwd.add(1)}
            else:
                st = {"amax": torch.zeros(3, dtype=torch.float32, device=dev),
                      "scale": torch.ones(3, dtype=torch.float32, device=dev),
                      "scale_inv": torch.ones(3, dtype=torch.float32, device=dev)}
            self._fp8[key] = st
        if key[0] == "delayed":
            f, b, i, j = st["pool"].fwd, st["pool"].bwd, st["fwd"], st["bwd"]
            return ((f.scale[i:i + 1], f.scale_inv[i:i + 1], f.hist[i, 0:1]),
                    (f.scale[i + 1:i + 2], f.scale_inv[i + 1:i + 2], f.hist[i + 1, 0:1]),
                    (b.scale[j:j + 1], b.scale_inv[j:j + 1], b.hist[j, 0:1]))
        return tuple((st["scale"][k:k + 1], st["scale_inv"][k:k + 1], st["amax"][k:k + 1]) for k in range(3))

    def fp8_state_dict(self, recipe=None):
        """The delayed-scaling state of this module (input, weight, output gradient) as
        plain tensors: amax_history [3, L], scale [3], scale_inv [3]."""
        st = self._delayed_state(recipe)
        if st is None:
            return {}
        f, b, i, j = st["pool"].fwd, st["pool"].bwd, st["fwd"], st["bwd"]
        return {"amax_history": torch.cat([f.hist[i:i + 2], b.hist[j:j + 1]]).clone(),
                "scale": torch.cat([f.scale[i:i + 2], b.scale[j:j + 1]]).clone(),
                "scale_inv": torch.cat([f.scale_inv[i:i + 2], b.scale_inv[j:j + 1]]).clone()}

    def load_fp8_state_dict(self, sd, recipe=None):
        """Restore what fp8_state_dict returned (recipe: the DelayedScaling it was saved
        under; by default the default recipe with the saved history length)."""
        if not sd:
            return
        if recipe is None:
            recipe = DelayedScaling(amax_history_len=int(sd["amax_history"].shape[1]))
        self._slots(recipe)
        st = self._fp8[_recipe_key(recipe)]
        f, b, i, j = st["pool"].fwd, st["pool"].bwd, st["fwd"], st["bwd"]
        dev = self.weight.device
        h, s, si = (sd[k].to(dev) for k in ("amax_history", "scale", "scale_inv"))
        with torch.no_grad():
            f.hist[i:i + 2].copy_(h[0:2])
            b.hist[j:j + 1].copy_(h[2:3])
            f.scale[i:i + 2].copy_(s[0:2])
            b.scale[j:j + 1].copy_(s[2:3])
            f.scale_inv[i:i + 2].copy_(si[0:2])
            b.scale_inv[j:j + 1].copy_(si[2:3])

    def _delayed_state(self, recipe):
        if not self._fp8:
            return None
        if recipe is not None:
            return self._fp8.get(_recipe_key(recipe))
        for k, v in self._fp8.items():
            if k[0] == "delayed":
                return v
        return None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        st = _current()
        bias = self.bias
        if st is not None and st.enabled:
            if isinstance(st.recipe, DelayedScaling):
                self._slots(st.recipe)
                pool = self._fp8[_recipe_key(st.recipe)]["pool"]
                st.pools[id(pool)] = pool
            need_grad = torch.is_grad_enabled() and (x2.requires_grad or self.weight.requires_grad)
            y = _FP8LinearFn.apply(x2, self.weight, bias, self, st.recipe, need_grad)
        else:
            xb = x2.to(torch.bfloat16).contiguous()
            wb = self.weight.to(torch.bfloat16).contiguous()
            y = torch.empty((x2.shape[0], self.out_features), dtype=torch.bfloat16, device=x.device)
            B.te_fp8_gemm(xb, "BF16", None, wb, "BF16", None, y, bias=bias)
        return y.reshape(*lead, self.out_features)
