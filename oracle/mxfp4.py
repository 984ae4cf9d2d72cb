"""MXFP4 expert store decoding and the NVFP4 scale-split check (FORMAT F9, F13).

Source passages:
- DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores" table (mxfp4 row: FP4 E2M1 values, one
  E8M0 scale per 32 inputs, 348,160 bytes per unit) and the paragraph under it (a native
  unit is its channels' source codes followed by their scales, HF orientation);
- DeepSeek-V4.1-Flash-1017 NVFP4 page, "Model" (the 16-element blocks refine the 32-element
  blocks; both halves inherit the source scale through weight_scale * weight_scale_2; the
  nibbles are unchanged; experts grow 5.9 %);
- the OCP Microscaling formats named in the K2 Mix page's credits: E2M1 elements with
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} (sign in bit 3) and E8M0 scales 2^(b-127),
  byte 255 = NaN.
"""

import math

import numpy as np

# E2M1 magnitudes by 3-bit code: exponent bits e (2), mantissa bit m (1);
# e = 0 is subnormal (m * 0.5), else 2^(e-1) * (1 + m/2).
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (bit 3 = sign, so code 8 is -0.0)."""
    if not 0 <= code < 16:
        raise ValueError("E2M1 code is 4 bits")
    mag = E2M1_VALUES[code & 7]
    return -mag if code & 8 else mag


def e8m0_value(b):
    """Value of an E8M0 scale byte: 2^(b-127); 255 is NaN."""
    if not 0 <= b < 256:
        raise ValueError("E8M0 is one byte")
    if b == 255:
        return math.nan
    return math.ldexp(1.0, b - 127)


def mxfp4_unit_bytes(out=128, inputs=5120):
    """Bytes of one MXFP4 unit: a nibble per weight plus a scale byte per 32 inputs."""
    assert inputs % 32 == 0
    return out * inputs // 2 + out * inputs // 32


def decode_mxfp4_unit(unit, out, inputs):
    """w[out, inputs] (float64) of one MXFP4 unit (FORMAT F9).

    Layout: codes uint8 [out][inputs/2] (element 2j = low nibble of byte j), then scales
    uint8 [out][inputs/32]. w = E2M1[code] * 2^(b - 127).
    """
    u = np.asarray(unit, dtype=np.uint8).reshape(-1)
    nc = out * inputs // 2
    if u.size != mxfp4_unit_bytes(out, inputs):
        raise ValueError("unit size does not match the shape")
    codes = u[:nc].reshape(out, inputs // 2)
    scales = u[nc:].reshape(out, inputs // 32)
    nib = np.empty((out, inputs), dtype=np.int64)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    table = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    vals = table[nib]
    sc = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)[scales]
    return vals * np.repeat(sc, 32, axis=1)


# ----------------------------------------------------------------------------------
# NVFP4 split (FORMAT F13): the closed form, and the oracle of the transcode kernel
# ----------------------------------------------------------------------------------

def e4m3_value(byte):
    """Value of an FP8 E4M3 byte (bias 7, no infinities, S.1111.111 = NaN)."""
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _e4m3_pow2_byte(k):
    """E4M3 byte for 2^k, k in [-9, 8] (normal for k >= -6, subnormal below)."""
    if -6 <= k <= 8:
        return (k + 7) << 3
    if -9 <= k < -6:
        return 1 << (k + 9)          # m/8 * 2^-6 = 2^k  ->  m = 2^(k+9)
    raise ValueError("2^%d is not exact in E4M3" % k)


def mxfp4_to_nvfp4(unit, out, inputs):
    """Split one MXFP4 unit's 32-blocks into NVFP4 16-blocks (FORMAT F13).

    Returns (nibble bytes unchanged, weight_scale E4M3 bytes [out][inputs/16],
    weight_scale_2 as float, lossless flag). Scales are anchored at the unit's largest
    exponent: weight_scale_2 = 2^(e_max - 8), weight_scale = 2^(e - e_max + 8).
    """
    u = np.asarray(unit, dtype=np.uint8).reshape(-1)
    nc = out * inputs // 2
    codes = u[:nc].copy()
    sb = u[nc:].reshape(out, inputs // 32).astype(np.int64)
    if np.any(sb == 255):
        raise ValueError("NaN scale has no NVFP4 form")
    e = sb - 127
    e_max = int(e.max())
    ws2 = math.ldexp(1.0, e_max - 8)
    rel = e - e_max + 8
    lossless = bool(np.all(rel >= -9))
    ws = np.zeros((out, inputs // 16), dtype=np.uint8)
    for o in range(out):
        for blk in range(inputs // 32):
            r = int(rel[o, blk])
            byte = _e4m3_pow2_byte(r) if r >= -9 else 0
            ws[o, 2 * blk] = byte
            ws[o, 2 * blk + 1] = byte
    return codes, ws, ws2, lossless


def decode_nvfp4(codes, ws, ws2, out, inputs):
    """w[out, inputs] of an NVFP4 tensor: E2M1[code] * E4M3(ws) * ws2, per 16-block."""
    c = np.asarray(codes, dtype=np.uint8).reshape(out, inputs // 2)
    nib = np.empty((out, inputs), dtype=np.int64)
    nib[:, 0::2] = c & 0x0F
    nib[:, 1::2] = c >> 4
    table = np.array([e2m1_value(k) for k in range(16)], dtype=np.float64)
    sc = np.array([[e4m3_value(int(b)) for b in row] for row in ws], dtype=np.float64)
    return table[nib] * np.repeat(sc, 16, axis=1) * ws2


def nvfp4_unit_bytes(out=128, inputs=5120):
    """Bytes of the NVFP4 form of a unit: nibbles plus one E4M3 byte per 16 inputs."""
    return out * inputs // 2 + out * inputs // 16
