"""CPU oracle for the per-tensor scaled FP8 (and MXFP8) linear-layer path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything in this package.  The
HIP library never calls it and it imports nothing from the HIP library: the two
sides share no code.  Inputs come from the seeded generators in
``fp8_precision_transformer_amd.synth`` (random numbers only, none of the
method's arithmetic).

Plain and slow on purpose: NumPy in float64 (exact for every FP8 product),
with each function citing the passage of the source pages it follows.

Pages cited (by title; section names are the pages' own headings):
  [TE-summary]  "NVIDIA Transformer Engine - 大規模Transformer向け高速低精度学習"
                (project summary page)
  [TE-readme]   "transformerengine" (README summary page)
  [FP8-intro]   "Introduction to FP8 training using Transformer Engine"
                (NVIDIA technical blog, Japanese edition)
  [LP-opt]      "How to Optimize Transformer-Based Models for Low-Precision
                Training" (NVIDIA technical blog, Japanese translation)

Parity status per function is stated in each module header.  Functions with
no pin other than a reading of the pages say "parity unpinned".
"""

from .formats import E4M3, E5M2, FP8Format, decode, decode_table, encode, fp8_format
from .quantize import (
    amax,
    current_scale,
    scale_inverse,
    scaled_cast,
    cast_transpose,
    DelayedScalingState,
    delayed_update,
    mxfp8_quantize,
    mx_scales_panel,
    mx_scales_from_panel,
    e8m0_to_float,
)
from .gemm import gemm_per_tensor, gemm_with_amax, gemm_mx, gemm_bf16, bf16_round_bits, bf16_bits_to_f32, rel_err, bias_grad
from .layernorm import layernorm
from .fp4_recipe import (hadamard, rht16_rows, philox4x64_10, sr_bits16, e2m1_encode_sr, mxfp4_quantize_sr,
                         mxfp4_quantize_2d)

__all__ = [
    "E4M3", "E5M2", "FP8Format", "decode", "decode_table", "encode", "fp8_format",
    "amax", "current_scale", "scale_inverse", "scaled_cast", "cast_transpose",
    "DelayedScalingState", "delayed_update", "mxfp8_quantize", "e8m0_to_float", "mx_scales_panel", "mx_scales_from_panel",
    "gemm_per_tensor", "gemm_with_amax", "gemm_mx", "gemm_bf16", "bf16_round_bits", "bf16_bits_to_f32",
    "rel_err", "bias_grad", "layernorm",
    "hadamard", "rht16_rows", "philox4x64_10", "sr_bits16", "e2m1_encode_sr", "mxfp4_quantize_sr",
    "mxfp4_quantize_2d",
]
