"""FP8 recipes.

[FP8-intro] "Transformer Engine の使い方": ``Format.HYBRID`` means E4M3 in the
forward pass and E5M2 in the backward pass; ``DelayedScaling(fp8_format,
amax_history_len, amax_compute_algo)`` carries the scaling-update settings.
[FP8-intro] "Transformer Engine 統合済みライブラリの利用" (NeMo keys): margin,
update interval, history length, ``max`` or ``most_recent``, ``fp8_wgrad``.
[LP-opt] "モデル設定とトレーニング入力" / "実モデルにおける結果の解釈": the
per-tensor current-scaling recipe and MXFP8 beside delayed scaling.

Defaults are readings where the pages show no default: history length 16 and
``max`` (the only explicit DelayedScaling call on the pages), margin 0 and
interval 1 (the NeMo example).
"""

from __future__ import annotations

from dataclasses import dataclass
from enum import Enum


class Format(Enum):
    E4M3 = "E4M3"      # E4M3 for every tensor
    HYBRID = "HYBRID"  # E4M3 forward (activations, weights), E5M2 backward (gradients)

    def forward_dtype(self) -> str:
        return "E4M3"

    def backward_dtype(self) -> str:
        return "E5M2" if self is Format.HYBRID else "E4M3"


@dataclass(frozen=True)
class DelayedScaling:
    fp8_format: Format = Format.HYBRID
    amax_history_len: int = 16
    amax_compute_algo: str = "max"  # or "most_recent"
    margin: int = 0
    interval: int = 1
    fp8_wgrad: bool = True

    def __post_init__(self):
        if self.amax_compute_algo not in ("max", "most_recent"):
            raise ValueError("amax_compute_algo must be 'max' or 'most_recent'")
        if self.interval != 1:
            raise NotImplementedError("only a scaling update interval of 1 is implemented")
        if self.amax_history_len < 1:
            raise ValueError("amax_history_len must be >= 1")


@dataclass(frozen=True)
class Float8CurrentScaling:
    fp8_format: Format = Format.HYBRID
    margin: int = 0
    fp8_wgrad: bool = True


@dataclass(frozen=True)
class MXFP8BlockScaling:
    fp8_format: Format = Format.E4M3  # E4M3 elements for every operand
    block: int = 32
