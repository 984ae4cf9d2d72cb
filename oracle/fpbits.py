"""Bit-level float helpers for the oracle (FORMAT F8, F10).

bf16 is the upper half of an IEEE binary32; f16 is IEEE binary16. These helpers turn
stored bit patterns into exact FP64 values and perform the one rounding the method
defines (fp32 -> bf16, round to nearest, ties to even).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits):
    """Exact value of IEEE binary16 bit patterns as float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_bf16_bits_rne(x):
    """Round binary32 values to bf16, nearest-even (FORMAT F8's last step).

    The upper 16 bits are kept; the lower 16 bits decide the rounding: above half an
    ulp rounds up, below rounds down, exactly half rounds to the even upper half.
    NaN stays NaN (quiet, sign kept).
    """
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    upper = u >> 16
    lower = u & 0xFFFF
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    out = (upper + round_up.astype(np.uint64)) & 0xFFFF
    nan = np.isnan(a)
    out = np.where(nan, (upper & 0x8000) | 0x7FC0, out)
    return out.astype(np.uint16)


def f64_to_bf16_bits_exact(x):
    """bf16 bit patterns of FP64 values that bf16 represents exactly (decoded weights).

    Raises if any value would need rounding; NaN maps to the canonical 0x7FC0.
    """
    a = np.asarray(x, dtype=np.float64)
    f = a.astype(np.float32)
    finite = ~np.isnan(a)
    if np.any(f[finite].astype(np.float64) != a[finite]):
        raise ValueError("value not exact in binary32")
    u = f.view(np.uint32)
    if np.any((u[finite] & 0xFFFF) != 0):
        raise ValueError("value not exact in bf16")
    out = (u >> 16).astype(np.uint16)
    return np.where(finite, out, np.uint16(0x7FC0)).astype(np.uint16)
