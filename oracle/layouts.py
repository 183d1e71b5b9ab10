"""Batched expert layout and row-wise ("fp8r") scales (test oracle).

Test infrastructure: see the package docstring for who may import this.

* Batched experts.  The "Fine-grained FP8" page of the transformers docs
  ("UE8M0 scale format") names two expert back-ends that take fp32 scales
  directly, ``grouped_mm`` and ``batched_mm``.  The grouped layout is
  :func:`oracle.gemm.grouped_block_gemm` (ragged experts packed row after
  row).  The batched layout is read as: every expert owns a fixed-capacity
  slab of C rows, x_q [E, C, K] with scales [E, C, K/128], of which the
  first count[e] rows hold tokens; y [E, C, N] is defined on those rows
  only (the rest are NaN here and left unwritten by the GPU).  count[e] is
  clamped to [0, C].
* Row-wise FP8 ("BFL (fp8r / nvfp4)" page of the diffusers docs,
  introduction: one fp32 weight scale per row, activations quantized per
  row at run time; "Kernels": a row-scaled fp8 matrix product).  The element
  map is that of the block scheme with the set = one whole row of K values:
  s = fl32(amax_row / 448), q = E4M3_RNE(fl32(x / s)), all-zero rows get
  s = 0.  The GEMM applies the scale pair once, outside the K sum:
      y[m,n] = s_x[m] * s_w[n] * sum_k dec(x_q[m,k]) * dec(w_q[n,k]).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import decode
from .gemm import block_gemm, term_magnitude
from .quant import quant_element_map


def batched_block_gemm(x_q, x_s, w_q, w_s, counts) -> np.ndarray:
    """x_q [E,C,K], x_s [E,C,K/128], w_q [E,N,K], w_s [E,ceil(N/128),K/128],
    counts [E] -> fp64 y_hat [E,C,N] (NaN on rows past count[e])."""
    E, C, K = x_q.shape
    N = w_q.shape[1]
    y = np.full((E, C, N), np.nan)
    for e in range(E):
        c = int(min(max(int(counts[e]), 0), C))
        if c:
            y[e, :c] = block_gemm(x_q[e, :c], x_s[e, :c], w_q[e], w_s[e])
    return y


def batched_term_magnitude(x_q, x_s, w_q, w_s, counts) -> np.ndarray:
    E, C, K = x_q.shape
    N = w_q.shape[1]
    S = np.full((E, C, N), np.nan)
    for e in range(E):
        c = int(min(max(int(counts[e]), 0), C))
        if c:
            S[e, :c] = term_magnitude(x_q[e, :c], x_s[e, :c], w_q[e], w_s[e])
    return S


def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rowwise_quant(bits):
    """Rows of bf16 bits [R, K] -> (codes uint8 [R, K], fp32 scales [R]);
    the same map serves weights (one scale per output row) and activations
    (one scale per token)."""
    v = _bf16_to_f32(np.asarray(bits, np.uint16))
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    R, K = v.shape
    amax = np.max(np.abs(v), axis=1, keepdims=True) if K else np.zeros((R, 1), np.float32)
    q, s = quant_element_map(v, amax)
    return q, s.reshape(R)


def rowwise_gemm(x_q, x_s, w_q, w_s) -> np.ndarray:
    """Unrounded fp64 y_hat[M,N] = s_x[m] s_w[n] sum_k dec(x_q) dec(w_q)."""
    P = decode(x_q) @ decode(w_q).T
    return np.asarray(x_s, np.float64)[:, None] * np.asarray(w_s, np.float64)[None, :] * P


def rowwise_term_magnitude(x_q, x_s, w_q, w_s) -> np.ndarray:
    P = np.abs(decode(x_q)) @ np.abs(decode(w_q)).T
    return np.abs(np.asarray(x_s, np.float64))[:, None] * np.abs(np.asarray(w_s, np.float64))[None, :] * P
