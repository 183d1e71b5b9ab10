"""CPU oracle for the fine-grained (block-scaled) FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this
code; only the tests, the smoke check and the CPU-baseline leg of the
benchmark may call it.  It shares no code, tables or constants with the HIP
path: the E4M3 codec here is written from the format's bit definition with
integer arithmetic, the quantizers follow the per-block / per-group
definition element by element, and the GEMM dequantizes to fp64 and calls a
plain fp64 matrix product.

What is computed, and where it comes from:

* Weights: one scale per 2D block of 128x128, 8-bit codes
  ("Fine-grained FP8" page of the transformers docs, introduction: weights
  are reduced to 8 bits per 2D block, ``weight_block_size=(128, 128)``).
* Activations: one scale per token per group of input channels, the group
  matching the weight block along the input channel (128 by default)
  (same page, introduction), computed at run time
  (same page, "DeepGEMM fast path": ``activation_scheme="dynamic"``).
* Scales are fp32 (same page, "UE8M0 scale format": ``float32`` is the
  default scale type that UE8M0 checkpoints replace).
* The linear layer's result is that of dequantize-then-matmul
  ("BFL (fp8r / nvfp4)" page of the diffusers docs, "Kernels": the
  device-independent path dequantizes the weights and runs a plain linear).
* The 8-bit format is OCP FP8 E4M3FN (bias 7, largest finite 448, NaN at
  S.1111.111, no infinities); encoding rounds to nearest, ties to even, and
  saturates at +-448; the scale of a block or group is fl32(amax / 448) and
  is the dequantization multiplier.  These are this library's readings of
  what the pages leave open.

* Power-of-two scales stored as E8M0 bytes ("UE8M0 scale format" on the
  same page, ``scale_fmt="ue8m0"``): :mod:`oracle.ue8m0` states the
  readings (codec, round-up exponent, activations scaled the same way).

* Static activation scales (same page, "DeepGEMM fast path": the static
  activation scheme): :mod:`oracle.static` states the readings (one
  calibrated fp32 scale per tensor, saturating quotient).

* The batched expert layout and row-wise ("fp8r") scales:
  :mod:`oracle.layouts` states the readings.

* SwiGLU ahead of the activation quantizer (the input of a mixture-of-
  experts down projection): :mod:`oracle.swiglu` states the readings.

Modules: :mod:`oracle.e4m3` (codec), :mod:`oracle.quant` (quantizers),
:mod:`oracle.gemm` (block-scaled and grouped GEMM, linear layer),
:mod:`oracle.ue8m0` (E8M0 scales: codec, quantizers, GEMM),
:mod:`oracle.static` (static activation scale: quantizer, GEMM),
:mod:`oracle.layouts` (batched experts; row-wise quantizer and GEMM),
:mod:`oracle.swiglu` (SwiGLU then the activation quantizer).
"""
from .e4m3 import E4M3_MAX, decode, encode, fl32_div
from .quant import act_quant_group, weight_block_quant, quant_element_map
from .gemm import (bf16_rne_bits, block_gemm, dequant_act, dequant_weight,
                   grouped_block_gemm, grouped_term_magnitude, linear, term_magnitude,
                   tolerance_report)
from .ue8m0 import (act_quant_group_ue8m0, block_gemm_ue8m0, e8m0_decode, e8m0_exponent,
                    grouped_block_gemm_ue8m0, weight_block_quant_ue8m0)
from .static import act_quant_static, block_gemm_static
from .layouts import batched_block_gemm, rowwise_gemm, rowwise_quant
from .swiglu import swiglu_act_quant, swiglu_act_quant_ue8m0, swiglu_bf16

__all__ = [
    "E4M3_MAX", "decode", "encode", "fl32_div",
    "act_quant_group", "weight_block_quant", "quant_element_map",
    "bf16_rne_bits", "block_gemm", "dequant_act", "dequant_weight",
    "grouped_block_gemm", "grouped_term_magnitude", "linear", "term_magnitude",
    "tolerance_report",
    "act_quant_group_ue8m0", "block_gemm_ue8m0", "e8m0_decode", "e8m0_exponent",
    "grouped_block_gemm_ue8m0", "weight_block_quant_ue8m0",
    "act_quant_static", "block_gemm_static",
    "batched_block_gemm", "rowwise_gemm", "rowwise_quant",
    "swiglu_act_quant", "swiglu_act_quant_ue8m0", "swiglu_bf16",
]
