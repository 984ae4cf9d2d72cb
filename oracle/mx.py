"""FP8 (E4M3) operands for the FP8 matrix-core variants (FORMAT F18).

Source passages: DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix page, "Credits" (the trellis
decoded directly into FP8 E4M3 tensor-core operands); DeepSeek-V4.1-Flash-1017 · exlr8
page, "Stores" (OCP MX block scaling: E8M0 scales per 32 elements, the official store's
format); the OCP Microscaling (MX) formats (credited on the K2 Mix page).

TEST INFRASTRUCTURE (see the package docstring). Written from the definitions:
- E4M3 (OCP "E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
  exponent field 0, no infinities, S.1111.111 = NaN, largest finite 448;
- rounding to E4M3: the nearest representable value, ties to the even code;
- MXFP8 activation blocks: each 32 consecutive inputs of a row share one E8M0 scale
  2^(b - 127), chosen so that the block's largest magnitude divided by it lies in
  [128, 256) (so no element can exceed 448); the elements are the E4M3 roundings of the
  scaled values;
- T16 values as E4M3 operands (FORMAT F19): the integer q of the T16 hash rounded to the
  nearest E4M3 value, its per-channel fp16 scale applied after the contraction as for the
  exact operands.
"""

import math

import numpy as np

from .mxfp4 import e4m3_value

E4M3_MAX = 448.0


def e4m3_all_values():
    """The 256 E4M3 codes' values (NaN for 0x7F and 0xFF), float64 [256]."""
    return np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_round(x):
    """Nearest E4M3 code of each value (ties to the even code), uint8.

    Magnitudes above 448 have no E4M3 code here (the callers never produce them) and
    raise; NaN gives the NaN code with the value's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    vals = e4m3_all_values()
    pos = np.arange(0, 0x7F)                      # codes of the non-negative finite values
    grid = vals[pos]                              # increasing: 0, 2^-9, ..., 448
    a = np.abs(x)
    fin = np.isfinite(a)
    if np.any(a[fin] > E4M3_MAX):
        raise ValueError("magnitude above 448 has no E4M3 code")
    a_f = np.where(fin, a, 0.0)
    hi = np.searchsorted(grid, a_f, side="left")  # first grid value >= a
    hi = np.minimum(hi, grid.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_f - grid[lo]
    d_hi = grid[hi] - a_f
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((pos[hi] & 1) == 0))
    code = np.where(pick_hi, pos[hi], pos[lo]).astype(np.uint8)
    code = np.where(a_f == grid[hi], pos[hi], code).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    out = code | sign
    return np.where(fin, out, sign | 0x7F).astype(np.uint8)


def mx_block_scale(amax):
    """E8M0 byte of a block with largest magnitude amax: amax / 2^(b - 127) in [128, 256),
    i.e. b = floor(log2 amax) - 7 + 127, kept in [0, 254]; 127 for an all-zero block; 255
    (NaN) for a non-finite amax."""
    if not math.isfinite(amax):
        return 255
    if amax == 0.0:
        return 127
    _, e = math.frexp(amax)                      # amax = f 2^e, f in [0.5, 1)
    return int(min(max((e - 1) - 7 + 127, 0), 254))


def quantize_mxfp8_rows(x_vals, block=32):
    """(codes uint8 [rows, n], scales uint8 [rows, n / 32]) of the MXFP8 form of each row."""
    x = np.asarray(x_vals, dtype=np.float64)
    rows, n = x.shape
    if n % block:
        raise ValueError("n must be a multiple of the block size")
    xb = x.reshape(rows, n // block, block)
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(xb), axis=2)
    amax = np.where(np.any(~np.isfinite(xb), axis=2), np.inf, amax)
    scales = np.vectorize(mx_block_scale, otypes=[np.uint8])(amax)
    factor = np.ldexp(1.0, 127 - scales.astype(np.int64))      # 2^(127 - b), exact
    scaled = xb * factor[:, :, None]
    scaled = np.where(scales[:, :, None] == 255, np.nan, scaled)
    codes = e4m3_round(scaled).reshape(rows, n)
    return codes, scales


def dequantize_mxfp8_rows(codes, scales, block=32):
    """Values of MXFP8 rows: E4M3(code) * 2^(b - 127); a NaN scale gives NaN."""
    vals = e4m3_all_values()[np.asarray(codes, dtype=np.uint8)]
    rows, n = vals.shape
    s = np.asarray(scales, dtype=np.int64)
    factor = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return (vals.reshape(rows, n // block, block) * factor[:, :, None]).reshape(rows, n)


def t16_e4m3(q):
    """E4M3 operand of T16 values (FORMAT F19): each integer q in [-255, 255] rounded to the
    nearest E4M3 value (ties to the even code). Returns the values, float64."""
    q = np.asarray(q)
    if np.any(np.abs(q) > 255):
        raise ValueError("T16 values lie in [-255, 255]")
    return e4m3_all_values()[e4m3_round(q.astype(np.float64))]


def t16_e4m3_codes(q):
    """E4M3 codes (uint8) of T16 values, as t16_e4m3 rounds them."""
    q = np.asarray(q)
    if np.any(np.abs(q) > 255):
        raise ValueError("T16 values lie in [-255, 255]")
    return e4m3_round(q.astype(np.float64))


def mxfp8_values(x_vals):
    """The values the FP8 matrix cores see for activation rows: MXFP8 quantisation (F18)
    followed by its exact decode."""
    codes, scales = quantize_mxfp8_rows(x_vals)
    return dequantize_mxfp8_rows(codes, scales)
