"""MXFP4 -> NVFP4 transcode on the GPU vs the oracle's scale split (FORMAT F13), bit for bit:
the nibbles, every 16-block's E4M3 scale byte, the unit's fp32 second-level scale and the
exactness flag."""

import numpy as np
import pytest

import oracle
from gpu_helpers import gpu, needs_gpu, ops, to_dev, torch
from workloads import mxfp4_decode_layer, mxfp4_layer, rng_for

pytestmark = [gpu, needs_gpu]


def transcode(layer_h):
    o = ops()
    L = o.Mxfp4Layer.from_host(layer_h)
    codes, scales, scale2, status = o.mxfp4_to_nvfp4(L)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), scales.cpu().numpy(), scale2.cpu().numpy(),
            status.cpu().numpy())


def unit_of(layer_h, e):
    out, inp = layer_h["out"], layer_h["in"]
    ub = oracle.mxfp4_unit_bytes(out, inp)
    return layer_h["units"][e * ub:(e + 1) * ub]


def check_unit(layer_h, e, codes, scales, scale2, status):
    out, inp = layer_h["out"], layer_h["in"]
    oc, ows, ows2, lossless = oracle.mxfp4_to_nvfp4(unit_of(layer_h, e), out, inp)
    assert np.array_equal(codes[e], oc), e
    assert np.array_equal(scales[e].reshape(out, inp // 16), ows), e
    assert scale2[e] == np.float32(ows2), (e, scale2[e], ows2)
    assert status[e] == (1 if lossless else 0), e


def test_small_layer_every_unit():
    layer = mxfp4_layer(600, 6, 32, 1024)
    got = transcode(layer)
    for e in range(6):
        check_unit(layer, e, *got)
    assert np.all(got[3] == 1)


def test_lossy_units_and_extreme_exponents():
    out, inp, E = 16, 512, 4
    layer = mxfp4_layer(601, E, out, inp)
    nc = out * inp // 2
    units = layer["units"].reshape(E, -1)
    rng = rng_for(601, 9)
    # unit 0: exponents over the whole E8M0 range (most blocks flush);
    # unit 1: spread of exactly 17 (still exact); unit 2: spread of 18 (one block flushes);
    # unit 3: the largest byte is 254 and the smallest 0 (scale2 = 2^119)
    units[0, nc:] = rng.integers(0, 255, size=out * inp // 32, dtype=np.uint8)
    units[1, nc:] = 100
    units[1, nc + 7] = 117
    units[2, nc:] = 100
    units[2, nc + 5] = 118
    units[3, nc:] = 3
    units[3, nc + 1] = 254
    units[3, nc + 2] = 0
    got = transcode(layer)
    for e in range(E):
        check_unit(layer, e, *got)
    assert list(got[3]) == [0, 1, 0, 0]


def test_small_exponents_give_subnormal_scale2():
    # bmax <= 8: 2^(bmax - 135) is an fp32 subnormal
    out, inp = 16, 512
    layer = mxfp4_layer(602, 2, out, inp)
    nc = out * inp // 2
    units = layer["units"].reshape(2, -1)
    units[0, nc:] = 0
    units[1, nc:] = 8
    units[1, nc + 3] = 1
    got = transcode(layer)
    for e in range(2):
        check_unit(layer, e, *got)
    assert got[2][0] == np.float32(2.0 ** -135) and got[2][1] == np.float32(2.0 ** -127)


def test_nan_scale_is_flagged():
    # A NaN byte (255) has no NVFP4 form: its blocks get the E4M3 NaN 0x7F, the unit status 2;
    # the other blocks are anchored at the largest non-NaN byte, i.e. they equal the split of
    # the same unit with the NaN byte replaced by the unit's smallest byte.
    out, inp = 16, 512
    layer = mxfp4_layer(603, 1, out, inp)
    nc = out * inp // 2
    units = layer["units"].reshape(1, -1)
    units[0, nc + 9] = 255
    got = transcode(layer)
    codes, scales, scale2, status = got
    assert status[0] == 2
    clean = units[0].copy()
    clean[nc + 9] = clean[nc:].min()
    oc, ows, ows2, _ = oracle.mxfp4_to_nvfp4(clean, out, inp)
    want = ows.reshape(-1).copy()
    want[18:20] = 0x7F
    assert np.array_equal(scales[0].reshape(-1), want)
    assert np.array_equal(codes[0], oc)
    assert scale2[0] == np.float32(ows2)


def test_full_size_layer_sampled_units():
    # the MXFP4 decode layer: 384 units of 128 x 5120; every status, 24 units checked in full
    layer = mxfp4_decode_layer()["layer"]
    got = transcode(layer)
    assert np.all(got[3] == 1)  # E8M0 bytes 119..125: every unit is exact
    for e in rng_for(604, 0).choice(layer["E"], size=24, replace=False):
        check_unit(layer, int(e), *got)
