"""Static activation quantization (test oracle).

Test infrastructure: see the package docstring for who may import this.

The "Fine-grained FP8" page of the transformers docs ("DeepGEMM fast path")
names a second activation scheme beside "dynamic": static activation
quantization, which its back-ends run on the Triton path.  The page gives no
arithmetic; this module fixes it as follows (the library's readings):

* One fp32 activation scale ``s`` per tensor, calibrated ahead of time and
  handed in (it is not derived from the data being quantized), with the
  same meaning as the dynamic scales: the dequantization multiplier,
  x ~= dec(q) * s.
* q = E4M3_RNE(sat(fl32(x / s))): the IEEE binary32 quotient, saturated to
  +-448 (inputs beyond the calibrated range clip -- the case the dynamic
  scheme never meets), then rounded to nearest even.  Signed zeros keep
  their sign.
* The GEMM is the block-scaled GEMM with that one scale in place of every
  per-token-group scale: y[m,n] = sum_kb s * w_s[n/128,kb] * P_kb[m,n].
"""
from __future__ import annotations

import numpy as np

from .e4m3 import encode, fl32_div
from .gemm import block_gemm, term_magnitude


def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def act_quant_static(x_bits, scale) -> np.ndarray:
    """x bf16 bits [M, K] and a positive finite fp32 scale -> codes uint8 [M, K]."""
    x = _bf16_to_f32(x_bits)
    s = np.float32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("the static scale must be positive and finite")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    t = fl32_div(x, s)
    # a quotient may overflow to +-inf for a tiny scale; saturation maps it to
    # +-448 like any other out-of-range value (encode clamps finite inputs)
    t = np.where(np.isinf(t), np.copysign(np.float32(448.0), t), t).astype(np.float32)
    return encode(t)


def block_gemm_static(x_q, scale, w_q, w_s) -> np.ndarray:
    """Unrounded fp64 y_hat with one activation scale for the whole tensor."""
    M, K = x_q.shape
    x_s = np.full((M, K // 128), np.float32(scale), dtype=np.float32)
    return block_gemm(x_q, x_s, w_q, w_s)


def term_magnitude_static(x_q, scale, w_q, w_s) -> np.ndarray:
    M, K = x_q.shape
    x_s = np.full((M, K // 128), np.float32(scale), dtype=np.float32)
    return term_magnitude(x_q, x_s, w_q, w_s)
