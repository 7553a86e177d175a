"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no scaling, no FP8 encoding, no GEMM).  Each tensor is
seeded by ``SeedSequence([cfg, layer, tensor_id, step])`` so the HIP path and the
oracle see identical bytes.

Distributions (no dataset is used; these stand in for the pages' workloads):
  * linear-layer example of [FP8-intro] "Transformer Engine の使い方":
    input ``torch.rand((1024, 768))`` -> U[0, 1) fp32; weight and bias N(0, 0.02);
  * BERT-base and CodonFM-5B shaped layers ([FP8-intro] "HuggingFace BERT を例にした
    Transformer Engine の適用", [LP-opt] "モデル設定とトレーニング入力"):
    activations N(0, 1) with exactly round(0.001 * numel) positions (uniform,
    without replacement) multiplied by 50; weights N(0, 0.02); output
    gradients Student-t(nu = 3) times 1e-3; all rounded to bf16 (round to
    nearest even, done by PyTorch's CPU conversion).

Large tensors are drawn in fixed 8 Mi-element chunks, each with its own child
seed, so the bytes do not depend on the number of worker threads.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 8 * 1024 * 1024

# tensor ids used in seeds
T_X, T_W, T_BIAS, T_DY = 0, 1, 2, 3


def generator(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _chunked(shape, key, fill):
    """Fill a float32 array chunk by chunk; fill(gen, out_slice) writes the slice in place."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, CHUNK))

    def work(ci):
        s = starts[ci]
        e = min(n, s + CHUNK)
        fill(generator(*key, ci), out[s:e])

    workers = max(1, min(8, os.cpu_count() or 1, len(starts)))
    if workers == 1:
        for ci in range(len(starts)):
            work(ci)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(len(starts))))
    return out.reshape(shape)


def uniform01(shape, *key) -> np.ndarray:
    return _chunked(shape, key, lambda g, o: g.random(dtype=np.float32, out=o))


def normal(shape, std, *key) -> np.ndarray:
    std = np.float32(std)

    def fill(g, o):
        g.standard_normal(dtype=np.float32, out=o)
        o *= std

    return _chunked(shape, key, fill)


def activations(shape, *key, outlier_frac=1e-3, outlier_mult=50.0) -> np.ndarray:
    """N(0,1) with exactly round(outlier_frac * numel) outliers multiplied by outlier_mult."""
    x = normal(shape, 1.0, *key)
    n = x.size
    k = int(round(outlier_frac * n))
    if k:
        g = generator(*key, 1 << 30)
        pos = g.choice(n, size=k, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(outlier_mult)
    return x


def grads(shape, *key, nu=3.0, scale=1e-3) -> np.ndarray:
    """Student-t(nu) times scale, sampled as sqrt(nu/2) * Z / sqrt(G) with Z ~ N(0,1) and
    G ~ Gamma(nu/2, 1) (the ratio of a normal and a chi-square root)."""
    c = np.float32(np.sqrt(nu / 2.0) * scale)

    def fill(g, o):
        g.standard_normal(dtype=np.float32, out=o)
        gam = np.empty_like(o)
        g.standard_gamma(nu / 2.0, dtype=np.float32, out=gam)
        np.maximum(gam, np.float32(1e-30), out=gam)  # a zero draw would give an infinite sample
        np.sqrt(gam, out=gam)
        o /= gam
        o *= c

    return _chunked(shape, key, fill)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (PyTorch CPU conversion) and return the uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact) for host-side consumers."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
