"""LayerNorm reference.

TEST INFRASTRUCTURE ONLY: imported by tests, __graft_entry__.smoke() and the
bench's CPU baseline, never by the library path.

[FP8-intro] "Transformer Engine の使い方" lists te.LayerNorm among the modules
that replace their PyTorch counterparts, and "HuggingFace BERT を例にした
Transformer Engine の適用" converts nn.LayerNorm(normalized_shape, eps) with its
weight and bias into te.LayerNorm; so the operation is nn.LayerNorm's:
normalization over the last axis with the biased variance,
    y = (x - mean) / sqrt(var + eps) * gamma + beta.
The oracle evaluates it in float64 (the exact result to float64 rounding) and
returns mean and 1/sqrt(var + eps) as well (the backward's saved statistics).

Pins (tests/test_oracle_layernorm.py): PyTorch's layer_norm on float64 CPU
tensors, constant rows (y = beta exactly), the zero-mean / variance invariants
of the normalized row, and a Python loop on a tiny input.
"""

from __future__ import annotations

import numpy as np


def layernorm(x, gamma, beta, eps):
    """(y, mean, rsigma), all float64: y[r, c] = (x[r, c] - mean[r]) * rsigma[r] * gamma[c] + beta[c]."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1)
    d = x - mean[:, None]
    var = (d * d).mean(axis=1)
    rsigma = 1.0 / np.sqrt(var + float(eps))
    y = d * rsigma[:, None] * np.asarray(gamma, np.float64)[None, :] + np.asarray(beta, np.float64)[None, :]
    return y, mean, rsigma
