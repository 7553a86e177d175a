"""GEMM shapes of one Transformer layer, derived from the model configuration.

[LP-opt] sections "モデル設定とトレーニング入力" and "autocast モードの使用と
事前量子化の比較": the benchmark tool takes hidden size, intermediate size,
heads, layers, micro-batch and sequence length; it computes the token count
M = micro_batch * seq (31 * 512 = 15,872 for CodonFM-5B) and derives the 12 GEMM
shapes: Fprop, Dgrad and Wgrad of the four weights (QKV projection, attention
output, MLP up, MLP down), each timed separately because the aspect ratio
changes which kernel is best.

Every GEMM is expressed in the TN form D[m, n] = A[m, k] . B[n, k]^T:
  Fprop  Y  = X  . W^T      -> (m, n, k) = (M, out, in)      A = X,    B = W
  Dgrad  dX = dY . W        -> (m, n, k) = (M, in, out)      A = dY,   B = W^T
  Wgrad  dW = dY^T . X      -> (m, n, k) = (out, in, M)      A = dY^T, B = X^T
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class ModelConfig:
    hidden_size: int
    intermediate_size: int
    num_attention_heads: int
    num_hidden_layers: int
    micro_batch_size: int
    sequence_length: int

    @property
    def tokens(self) -> int:
        return self.micro_batch_size * self.sequence_length


# [LP-opt] "モデル設定とトレーニング入力": CodonFM 5B
CODONFM_5B = ModelConfig(4096, 16384, 32, 24, 31, 512)
# BERT-base shaped block (hidden 768, intermediate 3072), 32 sequences of 128 tokens
BERT_BASE = ModelConfig(768, 3072, 12, 12, 32, 128)


@dataclass(frozen=True)
class Weight:
    name: str
    in_features: int
    out_features: int


@dataclass(frozen=True)
class GemmShape:
    weight: str
    stage: str  # "fprop" | "dgrad" | "wgrad"
    m: int
    n: int
    k: int

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


def layer_weights(cfg: ModelConfig):
    h, i = cfg.hidden_size, cfg.intermediate_size
    return [
        Weight("qkv", h, 3 * h),
        Weight("attn_out", h, h),
        Weight("mlp_up", h, i),
        Weight("mlp_down", i, h),
    ]


def layer_gemms(cfg: ModelConfig):
    """The 12 GEMMs of one layer, in (weight, stage) order."""
    M = cfg.tokens
    out = []
    for w in layer_weights(cfg):
        out.append(GemmShape(w.name, "fprop", M, w.out_features, w.in_features))
        out.append(GemmShape(w.name, "dgrad", M, w.in_features, w.out_features))
        out.append(GemmShape(w.name, "wgrad", w.out_features, w.in_features, M))
    return out


def layer_flops(cfg: ModelConfig) -> int:
    return sum(g.flops for g in layer_gemms(cfg))
