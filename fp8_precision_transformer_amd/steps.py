"""Whole steps of the FP8 linear-layer path, enqueued through the C ABI on one stream.

A step object owns its device buffers, its amax workspace included, and enqueues
every kernel of one step with ``run()``, so the same step can be timed eagerly or
captured once into a HIP graph and replayed (``capture``): the small configurations
are bound by launch latency, not by the kernels.  A graph captured from a step uses
that step's workspace, so it can be replayed on any stream while other work (with
its own workspace) runs beside it.

- ``LinearForwardStep``: the 768 -> 768 Linear layer of [FP8-intro] "Transformer
  Engine の使い方" on 1024 tokens of fp32 input, delayed scaling (history 16, max,
  margin 0, E4M3 for input and weight): amax+cast of X and W with last step's
  scales, the Fprop GEMM with bias (bf16 out), and the scaling update of both
  tensors ([FP8-intro] "FP8 のスケーリング": the history and the scale are updated
  after the step).
- ``LayerStep``: one transformer layer's four linear weights (QKV, attention out,
  MLP up, MLP down) with current scaling, HYBRID formats (E4M3 X and W, E5M2 dY),
  and the shared-quantization schedule: X, W and dY are each cast once into a row
  copy and a transposed copy, which Fprop, Dgrad and Wgrad reuse ([LP-opt]
  "autocast モードの使用と事前量子化の比較": Fprop, Dgrad and Wgrad are three
  GEMMs per weight).

Inputs come from the seeded generators in ``synth``; nothing here computes the
method's arithmetic on the host.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import synth
from .shapes import ModelConfig, layer_weights

E4, E5 = "E4M3", "E5M2"


def _bf16(x32: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(synth.to_bf16_bits(x32).view(np.int16)).to(dev).view(torch.bfloat16)


class LinearForwardStep:
    """One forward step of the 768 -> 768 Linear layer with delayed scaling."""

    def __init__(self, stream: torch.cuda.Stream, dev="cuda:0", tokens=1024, features=768, cfg_id=1):
        self.stream = stream
        t, f = tokens, features
        self.x = torch.from_numpy(synth.uniform01((t, f), cfg_id, 0, synth.T_X, 0)).to(dev)
        self.w = torch.from_numpy(synth.normal((f, f), 0.02, cfg_id, 0, synth.T_W, 0)).to(dev)
        self.b = torch.from_numpy(synth.normal((f,), 0.02, cfg_id, 0, synth.T_BIAS, 0)).to(dev)
        self.hist = torch.zeros((2, 16), dtype=torch.float32, device=dev)
        self.scale = torch.ones(2, dtype=torch.float32, device=dev)
        self.scale_inv = torch.ones(2, dtype=torch.float32, device=dev)
        self.xq = torch.empty((t, f), dtype=torch.uint8, device=dev)
        self.wq = torch.empty((f, f), dtype=torch.uint8, device=dev)
        self.y = torch.empty((t, f), dtype=torch.bfloat16, device=dev)
        self.ws = B.amax_workspace(dev)
        self.flops = 2 * t * f * f

    def reset(self):
        """Back to the initial scaling state (history 0, scale 1); eager only."""
        with torch.cuda.stream(self.stream):
            self.hist.zero_()
            self.scale.fill_(1.0)
            self.scale_inv.fill_(1.0)

    def run(self):
        s = self.stream
        B.te_amax_cast(self.x, E4, B.TE_SCALE_DELAYED, 0, self.scale[0:1], self.scale_inv[0:1],
                       self.hist[0, 0:1], self.xq, workspace=self.ws, stream=s)
        B.te_amax_cast(self.w, E4, B.TE_SCALE_DELAYED, 0, self.scale[1:2], self.scale_inv[1:2],
                       self.hist[1, 0:1], self.wq, workspace=self.ws, stream=s)
        B.te_fp8_gemm(self.xq, E4, self.scale_inv[0:1], self.wq, E4, self.scale_inv[1:2], self.y,
                      bias=self.b, stream=s)
        B.te_scale_update(self.hist, self.scale, self.scale_inv, E4, B.TE_AMAX_MAX, 0, stream=s)

    def outputs(self):
        return {"y": self.y, "xq": self.xq, "wq": self.wq, "hist": self.hist, "scale": self.scale,
                "scale_inv": self.scale_inv}


def splitk_splits(m: int, n: int, k_bytes: int, cus: int = 256, max_splits: int = 3) -> int:
    """k splits for a GEMM whose 256 x 256 tiles leave most compute units idle: enough
    workgroups to fill them, at least four 128-byte k stages per split, and at most
    `max_splits` (every split adds m * n fp32 partials to write and read back)."""
    tiles = -(-m // 256) * -(-n // 256)
    stages = -(-k_bytes // 128)
    return max(1, min(cus // tiles, stages // 4, max_splits))


class LayerStep:
    """Fprop, Dgrad and Wgrad of a layer's four linear weights, current scaling, each
    of X, W, dY cast once into row and transposed copies.  GEMMs with few output tiles
    (the Wgrad and Dgrad of a small layer) split k over more workgroups
    (te_fp8_gemm_splitk)."""

    def __init__(self, cfg: ModelConfig, stream: torch.cuda.Stream, dev="cuda:0", cfg_id=2):
        self.stream = stream
        self.cfg = cfg
        M = cfg.tokens
        self.weights = layer_weights(cfg)
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
        f1 = lambda: torch.ones(1, dtype=torch.float32, device=dev)  # noqa: E731
        self.t = {}
        self.ws = B.amax_workspace(dev)
        self.flops = 0
        for li, w in enumerate(self.weights):
            K, N = w.in_features, w.out_features
            self.t[w.name] = dict(
                X=_bf16(synth.activations((M, K), cfg_id, li, synth.T_X, 0), dev),
                W=_bf16(synth.normal((N, K), 0.02, cfg_id, li, synth.T_W, 0), dev),
                DY=_bf16(synth.grads((M, N), cfg_id, li, synth.T_DY, 0), dev),
                x=u8(M, K), xT=u8(K, M), w=u8(N, K), wT=u8(K, N), dy=u8(M, N), dyT=u8(N, M),
                sc={k: (f1(), f1(), f1()) for k in ("x", "w", "dy")},
                y=bf(M, N), dx=bf(M, K), dw=bf(N, K))
            self.flops += 3 * 2 * M * N * K
        # split-K plans (splits, workspace) of the Fprop, Dgrad and Wgrad GEMMs
        self.splits = {}
        for w in self.weights:
            K, N = w.in_features, w.out_features
            for stage, (m, n, k) in (("fprop", (M, N, K)), ("dgrad", (M, K, N)), ("wgrad", (N, K, M))):
                sp = splitk_splits(m, n, k)
                ws = u8(B.te_fp8_gemm_splitk_workspace_bytes(m, n, sp)) if sp > 1 else None
                self.splits[(w.name, stage)] = (sp, ws)

    def _gemm(self, key, a, fa, sa, b, fb, sb, d):
        sp, ws = self.splits[key]
        if sp > 1:
            B.te_fp8_gemm_splitk(a, fa, sa, b, fb, sb, d, sp, ws, stream=self.stream)
        else:
            B.te_fp8_gemm(a, fa, sa, b, fb, sb, d, stream=self.stream)

    def run(self):
        s, cur = self.stream, B.TE_SCALE_CURRENT
        for w in self.weights:
            t = self.t[w.name]
            sx, sw, sg = t["sc"]["x"], t["sc"]["w"], t["sc"]["dy"]
            B.te_cast_transpose(t["X"], E4, cur, 0, *sx, t["x"], t["xT"], workspace=self.ws, stream=s)
            B.te_cast_transpose(t["W"], E4, cur, 0, *sw, t["w"], t["wT"], workspace=self.ws, stream=s)
            self._gemm((w.name, "fprop"), t["x"], E4, sx[1], t["w"], E4, sw[1], t["y"])
            B.te_cast_transpose(t["DY"], E5, cur, 0, *sg, t["dy"], t["dyT"], workspace=self.ws, stream=s)
            self._gemm((w.name, "dgrad"), t["dy"], E5, sg[1], t["wT"], E4, sw[1], t["dx"])
            self._gemm((w.name, "wgrad"), t["dyT"], E5, sg[1], t["xT"], E4, sx[1], t["dw"])

    def outputs(self):
        out = {}
        for w in self.weights:
            t = self.t[w.name]
            for k in ("x", "xT", "w", "wT", "dy", "dyT", "y", "dx", "dw"):
                out[f"{w.name}.{k}"] = t[k]
            for k in ("x", "w", "dy"):
                out[f"{w.name}.scale_inv.{k}"] = t["sc"][k][1]
        return out


def capture(step) -> torch.cuda.CUDAGraph:
    """Capture one ``step.run()`` on the step's stream into a HIP graph (the step's
    buffers and workspace are allocated already, so the capture allocates nothing)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=step.stream, capture_error_mode="thread_local"):
        step.run()
    return g


def time_step(step, iters=50, warmup=5, graph=None) -> float:
    """Microseconds per step on the step's stream, eager or by graph replay."""
    s = step.stream
    with torch.cuda.stream(s):
        for _ in range(warmup):
            graph.replay() if graph is not None else step.run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(iters):
            graph.replay() if graph is not None else step.run()
        e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters
