"""Plain CPU decoding of OCP FP8 E4M3 bytes.

TEST INFRASTRUCTURE ONLY (see the package header).  The FP8 KV cache of the
decode step ("On-Policy Residual Learning for Diffusion Language Models",
paper cards page, Table 11 configurations) stores E4M3 values: one sign bit,
four exponent bits with bias 7, three mantissa bits, no infinities, and the
all-ones exponent-and-mantissa pattern as NaN.  A byte s.eeee.mmm is
  e > 0:  (-1)^s * 2^(e - 7) * (1 + m / 8)
  e = 0:  (-1)^s * 2^(-6) * (m / 8)
"""
from __future__ import annotations

import numpy as np


def e4m3_to_float(b) -> np.ndarray:
    """float64 values of E4M3 bytes (any integer array of 0..255)."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)
