"""OCP FP8 E4M3FN codec, written from the bit definition (test oracle).

Test infrastructure: see the package docstring for who may import this.

Format (OCP 8-bit floating point, E4M3 variant "FN"): sign s, 4 exponent
bits e (bias 7), 3 mantissa bits m.
  e == 0           -> (-1)^s * m * 2^-9              (subnormals, and +-0)
  1 <= e <= 15     -> (-1)^s * (1 + m/8) * 2^(e-7)
  e == 15, m == 7  -> NaN (0x7F, 0xFF); there are no infinities.
Largest finite magnitude 448 (0x7E), smallest normal 2^-6, smallest
subnormal 2^-9.

The pages call the format "8-bit" / "fp8" ("Fine-grained FP8" page,
introduction) without naming the variant; E4M3FN with saturation at +-448
is this library's reading.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_F32_448_BITS = 0x43E00000  # bit pattern of 448.0f


def decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + m.astype(np.float64) / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def encode(t) -> np.ndarray:
    """Finite fp32 values -> E4M3 codes (uint8).

    Clamp the magnitude to 448, then round to the nearest representable
    E4M3 value with ties to the even mantissa; the sign bit is kept, so -0
    and negative values that round to zero give 0x80.  Pure integer
    arithmetic on the fp32 bit pattern.
    """
    t = np.ascontiguousarray(t, dtype=np.float32)
    if not np.all(np.isfinite(t)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    bits = t.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) & 1
    mag = bits & 0x7FFFFFFF
    mag = np.minimum(mag, _F32_448_BITS)          # saturate: |t| > 448 -> 448
    E = mag >> 23                                  # biased fp32 exponent
    F = mag & 0x7FFFFF
    sig = np.where(E == 0, F, F | 0x800000)        # 24-bit integer significand
    Eeff = np.where(E == 0, 1, E)                  # value = sig * 2^(Eeff-150)
    ue = Eeff - 127                                # unbiased exponent of the binade
    eq = np.maximum(ue, -6)                        # E4M3 binade (subnormals share -6)
    # value / 2^(eq-3) = sig * 2^(Eeff-150-(eq-3)) = sig >> shift
    shift = (eq - 3) - (Eeff - 150)                # >= 20
    shift = np.minimum(shift, 40)
    n = sig >> shift
    rem = sig - (n << shift)
    half = np.int64(1) << (shift - 1)
    up = (rem > half) | ((rem == half) & ((n & 1) == 1))
    n = n + up.astype(np.int64)                    # count of quanta 2^(eq-3)
    # ue >= -6: code = (ue+7)<<3 | (n-8), and n == 16 carries into the
    # exponent; ue < -6: subnormal code n (n == 8 is the smallest normal).
    code = np.where(ue >= -6, (ue + 6) * 8 + n, n)
    code = np.where(n == 0, 0, code)
    code = code | (sign << 7)
    return code.astype(np.uint8)


def fl32_div(a, b) -> np.ndarray:
    """IEEE-754 binary32 quotient, round to nearest even (numpy's float32
    division is the IEEE operation; subnormals are kept)."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.divide(a, b, dtype=np.float32)
