"""Pins of the oracle's fp8b32 decoder (FORMAT F16) against the store size printed on the
exlr8 page, an independent E4M3 decoder (torch's float8_e4m3fn conversion), and the block
structure of the scales."""

import math

import numpy as np
import torch

import oracle
from workloads import fp8b32_layer, rng_for


def test_unit_size_matches_the_page(golden):
    sizes = {row[0]: row[1] for row in golden("store_sizes.txt")}
    assert oracle.fp8b32_unit_bytes(128, 5120) == int(sizes["fp8b32"])


def test_e4m3_against_torch():
    # every byte, decoded by the oracle's definition and by torch's float8_e4m3fn
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        v = oracle.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b] and math.copysign(1.0, v) == math.copysign(1.0, ref[b]), b


def test_block_scales_and_orientation():
    # one nonzero code per 32 x 32 block, each block with its own scale byte: the decoded
    # weight must sit at (row, column) of the code and carry that block's scale only
    out, inputs = 64, 96
    unit = np.zeros(oracle.fp8b32_unit_bytes(out, inputs), dtype=np.uint8)
    codes = unit[:out * inputs].reshape(out, inputs)
    scales = unit[out * inputs:].reshape(out // 32, inputs // 32)
    for bo in range(2):
        for bi in range(3):
            codes[32 * bo + 5 + bo, 32 * bi + 7 + bi] = 0x38          # 1.0
            scales[bo, bi] = 127 + 3 * bo + bi                        # 2^(3 bo + bi)
    w = oracle.decode_fp8b32_unit(unit, out, inputs)
    expect = np.zeros((out, inputs))
    for bo in range(2):
        for bi in range(3):
            expect[32 * bo + 5 + bo, 32 * bi + 7 + bi] = 2.0 ** (3 * bo + bi)
    assert np.array_equal(w, expect)


def test_vectorised_equals_scalar_definition():
    layer = fp8b32_layer(900, 1, 64, 128)
    u = layer["units"]
    w = oracle.decode_fp8b32_unit(u, 64, 128)
    rng = rng_for(900, 7)
    for o, i in zip(rng.integers(0, 64, 200), rng.integers(0, 128, 200)):
        s = oracle.decode_fp8b32_weight_scalar(u, 64, 128, int(o), int(i))
        assert (math.isnan(s) and math.isnan(w[o, i])) or s == w[o, i]


def test_nan_scale_and_nan_code():
    out, inputs = 32, 32
    unit = np.full(oracle.fp8b32_unit_bytes(out, inputs), 0x38, dtype=np.uint8)
    unit[-1] = 255                       # the only block's scale byte: NaN
    assert np.isnan(oracle.decode_fp8b32_unit(unit, out, inputs)).all()
    unit[-1] = 127
    unit[3] = 0x7F                       # E4M3 NaN code
    w = oracle.decode_fp8b32_unit(unit, out, inputs)
    assert np.isnan(w[0, 3]) and np.isnan(w).sum() == 1
