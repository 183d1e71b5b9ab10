"""SwiGLU followed by the activation quantizer (test oracle).

Test infrastructure: see the package docstring for who may import this.

In a mixture-of-experts layer the input of the down projection is the
SwiGLU of the gate/up projection's output, and the down projection is a
block-scaled FP8 GEMM like any other ("Fine-grained FP8" page of the
transformers docs: experts run through grouped back-ends with fp32 scales,
and activations are quantized per token per 128-channel group at run time,
"DeepGEMM fast path").  The pages do not spell SwiGLU out; this module
takes the textbook definition and the plainest layout (the library's
readings):

* The gate/up output of a token is one bf16 row of 2I values: the gate g in
  columns [0, I), the up value u in columns [I, 2I) (a merged gate/up weight
  [2I, K] with the gate rows first).
* h = SiLU(g) * u with SiLU(g) = g / (1 + e^-g), rounded once to bf16
  (nearest, ties to even) -- the value an unfused pipeline stores between
  the two steps.  Evaluated here in fp64 (the error of that evaluation is
  ~2^-52 relative, so the bf16 rounding is the exact value's rounding except
  within ~2^-52 of a rounding midpoint).
* The quantizer is then the per-token-group activation quantizer of
  :mod:`oracle.quant` applied to h [M, I] (I % 128 == 0).
* h must be finite (|SiLU(g) * u| below bf16's overflow threshold);
  anything else is outside the contract, as non-finite inputs are.
* With power-of-two scales (the "UE8M0 scale format" section of the same
  page) the quantizer is :func:`oracle.ue8m0.act_quant_group_ue8m0` on the
  same h.
"""
from __future__ import annotations

import numpy as np

from .gemm import bf16_rne_bits
from .quant import act_quant_group
from .ue8m0 import act_quant_group_ue8m0


def _bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def swiglu_bf16(gu_bits) -> np.ndarray:
    """gate/up bf16 bits [M, 2I] -> h bf16 bits [M, I]."""
    gu_bits = np.asarray(gu_bits, np.uint16)
    M, two_i = gu_bits.shape
    if two_i % 2:
        raise ValueError("the gate/up row must hold 2I values")
    I = two_i // 2
    v = _bf16_to_f64(gu_bits)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    g, u = v[:, :I], v[:, I:]
    with np.errstate(over="ignore"):
        e = np.exp(-g)                       # +inf for g < -709: SiLU(g) is then -0
    silu = g / (1.0 + e)
    h = silu * u
    out = bf16_rne_bits(h)
    if np.any((out & 0x7F80) == 0x7F80):
        raise ValueError("SiLU(g) * u overflows bf16: outside the contract")
    return out


def swiglu_act_quant(gu_bits):
    """gate/up bf16 bits [M, 2I] (I % 128 == 0) -> (codes uint8 [M, I],
    scales fp32 [M, I/128]) of h = bf16(SiLU(g) * u)."""
    return act_quant_group(swiglu_bf16(gu_bits))


def swiglu_act_quant_ue8m0(gu_bits):
    """As :func:`swiglu_act_quant` with E8M0 scale bytes [M, I/128]."""
    return act_quant_group_ue8m0(swiglu_bf16(gu_bits))
