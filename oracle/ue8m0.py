"""UE8M0 (power-of-two) scale format: codec, quantizers, GEMM (test oracle).

Test infrastructure: see the package docstring for who may import this.

The "Fine-grained FP8" page of the transformers docs ("UE8M0 scale format")
names a second scale type beside fp32: scales packed as
``float8_e8m0fnu``, selected by ``scale_fmt="ue8m0"``, as stored by
pre-quantized DeepSeek-V4-style checkpoints.  The page gives the type, not
the arithmetic; this module fixes it as follows (the library's readings):

* Codec.  E8M0 is the OCP MX scale type: 8 exponent bits, no sign, no
  mantissa, bias 127.  Byte b in [0, 254] encodes 2^(b - 127); 0xFF is NaN;
  there is no zero.  "Packed" is read as one byte per scale, in the same
  [rows, K/128] layout as the fp32 scales.
* Quantizer.  For a set (a 128x128 weight block or a 1x128 activation
  group) with amax = max |x|, the scale is the smallest power of two 2^e
  with amax <= 448 * 2^e, and never below 2^-127 (the smallest E8M0 value;
  an all-zero set therefore gets byte 0).  Rounding the scale up keeps
  every quotient inside E4M3's range, so no element saturates.
      q = enc(x / 2^e)       (the quotient is exact: a power-of-two scaling)
  Activations use power-of-two scales too, so that both operands of the
  GEMM carry E8M0 scales.
* GEMM.  Dequantize-then-matmul as for fp32 scales, with each scale byte
  decoded to its power of two.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import encode
from .gemm import block_gemm, grouped_block_gemm, grouped_term_magnitude, term_magnitude
from .quant import GROUP

E8M0_BIAS = 127
E8M0_NAN = 0xFF
E_MIN = -127                       # byte 0
_E4M3_MAX = 448.0


def e8m0_decode(b) -> np.ndarray:
    """E8M0 bytes -> float64 scales 2^(b - 127); NaN for 0xFF."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    v = np.exp2((b - E8M0_BIAS).astype(np.float64))
    return np.where(b == E8M0_NAN, np.nan, v)


def e8m0_exponent(amax) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (amax >= 0, finite,
    fp32).  448 * 2^e and amax are exact in float64, so every comparison
    below is exact; the log2 guess is only a starting point."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("amax must be finite and >= 0")
    with np.errstate(divide="ignore"):
        guess = np.ceil(np.log2(a / _E4M3_MAX))
    e = np.where(a > 0, guess, E_MIN)
    e = np.clip(np.nan_to_num(e, neginf=E_MIN), E_MIN, 200).astype(np.int64)
    for _ in range(2):  # repair a guess that log2's rounding put one off
        e = np.where(a > _E4M3_MAX * np.exp2(e.astype(np.float64)), e + 1, e)
        lower = (e > E_MIN) & (a <= _E4M3_MAX * np.exp2((e - 1).astype(np.float64)))
        e = np.where(lower, e - 1, e)
    return e


def quant_element_map_ue8m0(x_f32, amax_f32):
    """Values x (fp32, exactly bf16) in a set with the given amax
    (broadcastable) -> (codes uint8, scale bytes uint8)."""
    x = np.asarray(x_f32, dtype=np.float32).astype(np.float64)
    e = e8m0_exponent(amax_f32)
    t = x * np.exp2(-e.astype(np.float64))                # exact in float64
    # |t| <= 448; a t below fp32's range rounds to a signed zero, whose code
    # is the same as the exact value's (anything under 2^-10 encodes to 0).
    codes = encode(t.astype(np.float32))
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def act_quant_group_ue8m0(x_bits):
    """x bf16 bits [M, K] (K % 128 == 0) -> (codes uint8 [M, K],
    scale bytes uint8 [M, K/128]); group g of token m is columns
    [128g, 128g+128)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    x = _bf16_to_f32(x_bits).reshape(M, K // GROUP, GROUP)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    amax = np.max(np.abs(x), axis=2, keepdims=True) if M else np.zeros((0, K // GROUP, 1), np.float32)
    q, b = quant_element_map_ue8m0(x, amax)
    return q.reshape(M, K), b.reshape(M, K // GROUP)


def weight_block_quant_ue8m0(w_bits):
    """W bf16 bits [N, K] (K % 128 == 0) -> (codes uint8 [N, K],
    scale bytes uint8 [ceil(N/128), K/128]); blocks as for fp32 scales (the
    last block row covers only the rows that exist)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = _bf16_to_f32(w_bits)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite input is outside the contract")
    NB, KB = -(-N // GROUP), K // GROUP
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((NB, KB), dtype=np.uint8)
    for nb in range(NB):
        r0, r1 = nb * GROUP, min(N, nb * GROUP + GROUP)
        blk = w[r0:r1].reshape(r1 - r0, KB, GROUP)
        amax = np.max(np.abs(blk), axis=(0, 2))
        q, b = quant_element_map_ue8m0(blk, amax[None, :, None])
        codes[r0:r1] = q.reshape(r1 - r0, K)
        scales[nb] = b.reshape(KB)
    return codes, scales


def block_gemm_ue8m0(x_q, x_e, w_q, w_e) -> np.ndarray:
    """Unrounded fp64 y_hat[M,N] with E8M0 scale bytes on both operands."""
    return block_gemm(x_q, e8m0_decode(x_e), w_q, e8m0_decode(w_e))


def term_magnitude_ue8m0(x_q, x_e, w_q, w_e) -> np.ndarray:
    return term_magnitude(x_q, e8m0_decode(x_e), w_q, e8m0_decode(w_e))


def grouped_block_gemm_ue8m0(x_q, x_e, w_q, w_e, offsets) -> np.ndarray:
    return grouped_block_gemm(x_q, e8m0_decode(x_e), w_q, e8m0_decode(w_e), offsets)


def grouped_term_magnitude_ue8m0(x_q, x_e, w_q, w_e, offsets) -> np.ndarray:
    return grouped_term_magnitude(x_q, e8m0_decode(x_e), w_q, e8m0_decode(w_e), offsets)
