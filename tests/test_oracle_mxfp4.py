"""Pins of the oracle's MXFP4 decoder and NVFP4 split against the OCP MX tables and the
sizes / invariants printed on the exlr8 and NVFP4 pages."""

import math

import numpy as np

import oracle
from oracle.mxfp4 import _e4m3_pow2_byte
from workloads import mxfp4_layer


def test_e2m1_table(golden):
    for code, value in golden("ocp_mx_e2m1.txt")[:16]:
        v = oracle.e2m1_value(int(code))
        assert v == float(value)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(value))


def test_e8m0_and_e4m3(golden):
    for kind, byte, value in golden("ocp_mx_e2m1.txt")[16:]:
        b = int(byte, 0)
        v = oracle.e8m0_value(b) if kind == "e8m0" else oracle.e4m3_value(b)
        if value == "nan":
            assert math.isnan(v)
        else:
            assert v == float(value)


def test_e4m3_powers_of_two():
    for k in range(-9, 9):
        assert oracle.e4m3_value(_e4m3_pow2_byte(k)) == 2.0 ** k


def test_nibble_order_and_scale_rows():
    out, inputs = 2, 64
    codes = np.zeros((out, inputs // 2), dtype=np.uint8)
    codes[0, 0] = 0x71          # element 0 = code 1 (0.5), element 1 = code 7 (6.0)
    codes[1, 31] = 0x8A         # element 62 = code 0xA (-1.0), element 63 = code 8 (-0.0)
    scales = np.full((out, inputs // 32), 127, dtype=np.uint8)
    scales[1, 1] = 129          # row 1, inputs 32..63 scaled by 4
    unit = np.concatenate([codes.reshape(-1), scales.reshape(-1)])
    w = oracle.decode_mxfp4_unit(unit, out, inputs)
    assert w[0, 0] == 0.5 and w[0, 1] == 6.0
    assert w[1, 62] == -4.0
    assert w[1, 63] == 0.0 and math.copysign(1.0, w[1, 63]) == -1.0
    assert np.count_nonzero(w) == 3


def test_nan_scale():
    unit = np.zeros(32 // 2 + 1, dtype=np.uint8)
    unit[-1] = 255
    assert np.all(np.isnan(oracle.decode_mxfp4_unit(unit, 1, 32)))


def test_unit_size(golden):
    sizes = {row[0]: row[1] for row in golden("store_sizes.txt")}
    assert oracle.mxfp4_unit_bytes() == int(sizes["mxfp4"])
    # fp8b32: one E4M3 byte per weight plus one E8M0 per 32 x 32 block
    assert 128 * 5120 + 128 * 5120 // 1024 == int(sizes["fp8b32"])


def test_nvfp4_split_lossless_and_growth(golden):
    sizes = {row[0]: row[1] for row in golden("store_sizes.txt")}
    layer = mxfp4_layer(101, 2, 32, 256)
    units = layer["units"].reshape(2, -1)
    for u in units:
        codes, ws, ws2, lossless = oracle.mxfp4_to_nvfp4(u, 32, 256)
        assert lossless
        assert np.array_equal(codes, u[:32 * 128])          # nibbles unchanged
        a = oracle.decode_mxfp4_unit(u, 32, 256)
        b = oracle.decode_nvfp4(codes, ws, ws2, 32, 256)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))  # bit for bit, -0 kept
    growth = oracle.nvfp4_unit_bytes() / oracle.mxfp4_unit_bytes() - 1.0
    assert round(100 * growth, 1) == float(sizes["nvfp4_growth_percent"])


def test_nvfp4_split_not_lossless_beyond_range():
    out, inputs = 1, 64
    unit = np.zeros(out * inputs // 2 + 2, dtype=np.uint8)
    unit[:32] = 0x22
    unit[-2:] = [127 + 10, 127 - 10]      # exponent spread 20 > 17
    _, _, _, lossless = oracle.mxfp4_to_nvfp4(unit, out, inputs)
    assert not lossless
