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


# ---------------------------------------------------------------------------
# Device-side generators for the workloads too large to draw on the host every step
# (the 24-layer CodonFM-5B drift sweep): torch's seeded generator on the GPU, the same
# distributions as above, bf16 by round to nearest even.  The host side of a test copies
# what it needs (amax, sampled rows) back; both sides see identical bytes.
# ---------------------------------------------------------------------------

def _torch_seed(*key: int) -> int:
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def gpu_generator(device, *key):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*key))
    return g


def gpu_normal(shape, std, device, *key):
    """N(0, std) as bf16 on `device`."""
    import torch

    g = gpu_generator(device, *key)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * np.float32(std)).to(torch.bfloat16)


def gpu_activations(shape, device, *key, outlier_frac=1e-3, outlier_mult=50.0):
    """N(0, 1) with exactly round(outlier_frac * numel) positions (without replacement)
    multiplied by outlier_mult, as bf16 on `device`."""
    import torch

    g = gpu_generator(device, *key)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    n = x.numel()
    k = int(round(outlier_frac * n))
    if k:
        pos = torch.randperm(n, generator=g, device=device)[:k]
        x.view(-1)[pos] *= np.float32(outlier_mult)
    return x.to(torch.bfloat16)


def gpu_grads(shape, device, *key, scale=1e-3):
    """Student-t(3) times scale as bf16 on `device`: Z sqrt(3 / (Z1^2 + Z2^2 + Z3^2)), the
    ratio of a normal and the root of a chi-square with three degrees of freedom."""
    import torch

    g = gpu_generator(device, *key)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros_like(z)
    for _ in range(3):
        u = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi.addcmul_(u, u)
    chi.clamp_(min=1e-30)
    return (z * torch.rsqrt(chi / 3.0) * np.float32(scale)).to(torch.bfloat16)


def drift(x_bf16, step: int, rate: float = 1.05):
    """x * rate^step: an fp32 multiply by fl32(rate^step), then bf16 rounding (host or device
    tensor); the input scale of a training-like run that grows every step."""
    import torch

    return (x_bf16.float() * float(np.float32(rate ** step))).to(torch.bfloat16)
