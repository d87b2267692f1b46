"""bf16 decoding and rounding for the oracle (its own, shared with nothing).

bfloat16 is the upper half of an IEEE binary32: sign, 8 exponent bits and 7
stored mantissa bits (8 significant bits).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(arr) -> np.ndarray:
    """Weights arrive either as bf16 bit patterns (uint16) or as floats."""
    a = np.asarray(arr)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, returned as
    float64.  Direct rounding of the exact value: with x = m * 2^e and
    0.5 <= |m| < 1, the 8 significant bits are round_half_even(m * 2^8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.round(m * 256.0)  # numpy rounds halves to even
    return np.ldexp(r, e - 8)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), rounding to nearest even."""
    r = round_to_bf16(x).astype(np.float32)  # exact: r has 8 significant bits
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
