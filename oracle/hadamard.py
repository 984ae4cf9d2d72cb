"""128-wide Hadamard input rotation (FORMAT F8).

Source passages: DeepSeek-V4.1-Flash-1017 · dsx T16 page, "How T16 works" (opening
paragraph: 128-wide Hadamard rotations as incoherence processing); DeepSeek-V4.1-Flash-1017
· exlr8 page, "Stores" (a 128 x 128 Hadamard with per-layer signs shared by all encodes of
a layer).

Forms:
- ``hadamard128_f64``: the exact orthonormal transform H/sqrt(128) applied to s * x in
  FP64, H the Sylvester matrix in natural order (no rounding at all);
- ``hadamard128_fp32_order``: the rounding FORMAT F8 fixes for the bf16 output — seven
  fp32 butterfly stages (strides 1..64), times fp32(1/sqrt(128)), rounded to bf16;
- ``rotate128_values``: the exact transform of FP64 values (the rotation of the FFN's
  intermediate, FORMAT F15, which is not rounded);
- ``output_rotation128``: the output-side rotation of FORMAT F17, s * (H/sqrt(128)) y, the
  transpose of the input rotation (exlr8 page, "Stores": Hadamard on both sides).
"""

import numpy as np

from .fpbits import bf16_bits_to_f64, f32_to_bf16_bits_rne

BLOCK = 128
INV_SQRT128_F32 = np.uint32(0x3DB504F3).view(np.float32)


def sylvester_hadamard(n):
    """Unnormalised Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _check(x_bits, signs):
    x = np.asarray(x_bits, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("x must be [rows, n] with n a multiple of 128")
    if signs is None:
        s = np.ones(x.shape[1], dtype=np.int64)
    else:
        s = np.asarray(signs, dtype=np.int64).reshape(-1)
        if s.size != x.shape[1] or np.any((s != 1) & (s != -1)):
            raise ValueError("signs must be +-1, one per input channel")
    return x, s


def hadamard128_f64(x_bits, signs=None):
    """Exact rotation in FP64: per 128-block, (H / sqrt(128)) (s * x). Returns float64."""
    x, s = _check(x_bits, signs)
    v = bf16_bits_to_f64(x) * s[None, :]
    rows, n = v.shape
    h = sylvester_hadamard(BLOCK).astype(np.float64) / np.sqrt(128.0)
    blocks = v.reshape(rows, n // BLOCK, BLOCK)
    return np.einsum("ij,rbj->rbi", h, blocks).reshape(rows, n)


def hadamard128_fp32_order(x_bits, signs=None):
    """FORMAT F8 exactly: fp32 butterflies with strides 1, 2, ..., 64, each pair
    (a, b) -> (a + b, a - b); then x fp32 0x3DB504F3; then bf16 round-to-nearest-even.
    Returns bf16 bit patterns (uint16)."""
    x, s = _check(x_bits, signs)
    v = (bf16_bits_to_f64(x) * s[None, :]).astype(np.float32)  # sign flip is exact
    rows, n = v.shape
    v = v.reshape(rows, n // BLOCK, BLOCK)
    h = 1
    while h < BLOCK:
        g = v.reshape(rows, n // BLOCK, BLOCK // (2 * h), 2, h)
        a = g[:, :, :, 0, :]
        b = g[:, :, :, 1, :]
        v = np.stack([a + b, a - b], axis=3).reshape(rows, n // BLOCK, BLOCK)
        h *= 2
    v = (v * INV_SQRT128_F32).astype(np.float32)
    return f32_to_bf16_bits_rne(v.reshape(rows, n))


def _signs_for(n, signs):
    if signs is None:
        return np.ones(n, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64).reshape(-1)
    if s.size != n or np.any((s != 1) & (s != -1)):
        raise ValueError("signs must be +-1, one per channel")
    return s


def _blocks_times_h(v):
    rows, n = v.shape
    if n % BLOCK:
        raise ValueError("the last axis must be a multiple of 128")
    h = sylvester_hadamard(BLOCK).astype(np.float64) / np.sqrt(128.0)
    return np.einsum("ij,rbj->rbi", h, v.reshape(rows, n // BLOCK, BLOCK)).reshape(rows, n)


def rotate128_values(v, signs=None):
    """Input-side rotation of FP64 values, exact: per 128-block, (H / sqrt(128)) (s * v)."""
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1, shape[-1])
    return _blocks_times_h(v * _signs_for(shape[-1], signs)[None, :]).reshape(shape)


def output_rotation128(y, signs=None):
    """Output-side rotation (FORMAT F17), exact: per 128-block of the last axis,
    s * ((H / sqrt(128)) y). The transpose of rotate128_values with the same signs."""
    y = np.asarray(y, dtype=np.float64)
    shape = y.shape
    y = y.reshape(-1, shape[-1])
    return (_blocks_times_h(y) * _signs_for(shape[-1], signs)[None, :]).reshape(shape)
