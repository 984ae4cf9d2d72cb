"""fp8b32 expert store decoding (FORMAT F16).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source passages:
- DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores" table (fp8b32 row: the shared expert's
  store, FP8 E4M3 values with one E8M0 scale per 32 x 32 block, 656,000 bytes per unit)
  and the paragraph under it (a native unit is its channels' source codes followed by
  their scales, HF orientation), and the layout notes (the shared expert is expert E);
- the OCP 8-bit floating point format named alongside MX: E4M3 with bias 7, no
  infinities, S.1111.111 = NaN; E8M0 scales 2^(b-127), byte 255 = NaN.

Reading (the page gives the block size but not the byte order of the scales): a unit of
out x in weights is codes uint8 [out][in] (row = output channel) followed by E8M0 scales
uint8 [out/32][in/32], row-major; the weight at (o, i) is E4M3[code[o][i]] times
2^(b - 127) with b = scales[o // 32][i // 32]. For 128 x 5120 this is 655,360 + 640 =
656,000 bytes, the page's figure.
"""

import numpy as np

from .mxfp4 import e4m3_value, e8m0_value


def fp8b32_unit_bytes(out=128, inputs=5120):
    """Bytes of one fp8b32 unit: a byte per weight plus a scale byte per 32 x 32 block."""
    if out % 32 or inputs % 32:
        raise ValueError("fp8b32 units are whole 32 x 32 blocks")
    return out * inputs + (out // 32) * (inputs // 32)


def decode_fp8b32_unit(unit, out, inputs):
    """w[out, inputs] (float64) of one fp8b32 unit (FORMAT F16): E4M3[code] * 2^(b - 127)
    with b the scale byte of the weight's 32 x 32 block."""
    u = np.asarray(unit, dtype=np.uint8).reshape(-1)
    if u.size != fp8b32_unit_bytes(out, inputs):
        raise ValueError("unit size does not match the shape")
    nc = out * inputs
    codes = u[:nc].reshape(out, inputs)
    scales = u[nc:].reshape(out // 32, inputs // 32)
    table = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
    sc = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)[scales]
    return table[codes] * np.repeat(np.repeat(sc, 32, axis=0), 32, axis=1)


def decode_fp8b32_weight_scalar(unit, out, inputs, o, i):
    """One weight by the definition, for brute-force checks on small units."""
    u = np.asarray(unit, dtype=np.uint8).reshape(-1)
    code = int(u[o * inputs + i])
    b = int(u[out * inputs + (o // 32) * (inputs // 32) + i // 32])
    return e4m3_value(code) * e8m0_value(b)
