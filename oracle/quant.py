"""Block and group quantizers (test oracle).

Test infrastructure: see the package docstring for who may import this.

Both quantizers apply the same element map to a set of bf16 values that
share one scale:
    amax = max |x|                          (exact: bf16 widens exactly to fp32)
    s    = fl32(amax / 448)                 (fp32 scale = dequantization multiplier)
    q    = enc(fl32(x / s))                 (fp32 quotient first, then E4M3 RNE)
For a set whose values are all zero (amax = 0) the formula's 0/0 is read as:
s = 0 and every code is a signed zero carrying the input's sign bit.

* Weights: the set is a 2D block of 128x128 ("Fine-grained FP8" page,
  introduction, ``weight_block_size=(128, 128)``); the last block row may be
  shorter when N is not a multiple of 128 and then covers only the rows that
  exist.
* Activations: the set is one token's 128 consecutive input channels
  (same page, introduction: per token, per group, group = the weight block
  along the input channel, 128 by default), recomputed on every call
  (same page, "DeepGEMM fast path", ``activation_scheme="dynamic"``).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import encode, fl32_div

GROUP = 128
_F32_448 = np.float32(448.0)


def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quant_element_map(x_f32, amax_f32):
    """Element map for values ``x`` (fp32, exactly bf16) quantized in a set
    whose amax is ``amax`` (broadcastable).  Returns (codes uint8, s fp32)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.asarray(amax_f32, dtype=np.float32)
    s = fl32_div(amax, _F32_448)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    t = fl32_div(x, s_safe)
    t = np.where(np.broadcast_to(zero, t.shape), x, t)  # all-zero set: keep +-0
    return encode(t), s.astype(np.float32)


def act_quant_group(x_bits):
    """x bf16 bits [M, K] (K % 128 == 0) -> (codes uint8 [M, K],
    scales fp32 [M, K/128]); group g of token m is columns [128g, 128g+128)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    x = _bf16_to_f32(x_bits).reshape(M, K // GROUP, GROUP)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    amax = np.max(np.abs(x), axis=2, keepdims=True) if M else np.zeros((0, K // GROUP, 1), np.float32)
    q, s = quant_element_map(x, amax)
    return q.reshape(M, K), s.reshape(M, K // GROUP)


def weight_block_quant(w_bits):
    """W bf16 bits [N, K] (K % 128 == 0) -> (codes uint8 [N, K],
    scales fp32 [ceil(N/128), K/128]); block (nb, kb) is rows
    [128nb, min(N, 128nb+128)) x columns [128kb, 128kb+128)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = _bf16_to_f32(w_bits)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite input is outside the contract")
    NB, KB = -(-N // GROUP), K // GROUP
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((NB, KB), dtype=np.float32)
    for nb in range(NB):
        r0, r1 = nb * GROUP, min(N, nb * GROUP + GROUP)
        blk = w[r0:r1].reshape(r1 - r0, KB, GROUP)          # rows x kb x 128
        amax = np.max(np.abs(blk), axis=(0, 2))              # one per kb
        q, s = quant_element_map(blk, amax[None, :, None])
        codes[r0:r1] = q.reshape(r1 - r0, K)
        scales[nb] = s.reshape(KB)
    return codes, scales
