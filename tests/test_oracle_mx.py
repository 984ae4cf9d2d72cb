"""Pins of the FP8 operand oracle (FORMAT F18): the E4M3 value table and its rounding
against torch's float8_e4m3fn (an independent implementation of the OCP format), the round
trip of every code, the MX block scale's closed form, and the quantisation error bound."""

import math

import numpy as np
import pytest

import oracle
from workloads import rng_for

torch = pytest.importorskip("torch")


def test_e4m3_values_match_torch():
    vals = oracle.e4m3_all_values()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(vals), np.isnan(ref))
    ok = ~np.isnan(vals)
    assert np.array_equal(vals[ok], ref[ok])
    assert vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9


def test_every_code_rounds_to_itself():
    vals = oracle.e4m3_all_values()
    codes = np.array([c for c in range(256) if not math.isnan(vals[c])], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_round(vals[codes]), codes)


def test_rounding_matches_torch_on_ties_and_random_values():
    vals = oracle.e4m3_all_values()
    pos = np.sort(vals[(vals >= 0) & ~np.isnan(vals)])
    mids = (pos[1:] + pos[:-1]) / 2                        # exact ties (binary fractions)
    rng = rng_for(720, 0)
    rand = rng.uniform(-448, 448, 20000) * np.exp2(-rng.integers(0, 18, 20000))
    xs = np.concatenate([mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20), rand])
    xs = xs.astype(np.float32).astype(np.float64)          # values torch rounds from fp32
    got = oracle.e4m3_round(xs)
    ref = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_block_scale_closed_form():
    assert oracle.mx_block_scale(1.0) == 120            # 1 / 2^-7 = 128
    assert oracle.mx_block_scale(255.99) == 127
    assert oracle.mx_block_scale(256.0) == 128
    assert oracle.mx_block_scale(0.0) == 127
    assert oracle.mx_block_scale(float("inf")) == 255
    assert oracle.mx_block_scale(2.0 ** -140) == 0      # clamped at the smallest E8M0 scale
    rng = rng_for(720, 1)
    for a in rng.uniform(0, 1, 200) * np.exp2(rng.integers(-100, 100, 200)):
        b = oracle.mx_block_scale(float(a))
        assert 128 <= a / 2.0 ** (b - 127) < 256


def test_quantize_rows_error_bound_and_special_blocks():
    rng = rng_for(720, 2)
    x = rng.standard_normal((4, 256)) * np.exp2(rng.integers(-20, 20, (4, 1)))
    x[1, 32:64] = 0.0
    x[2, 64] = np.inf
    codes, scales = oracle.quantize_mxfp8_rows(x)
    back = oracle.dequantize_mxfp8_rows(codes, scales)
    assert scales[1, 1] == 127 and np.all(back[1, 32:64] == 0.0)
    assert scales[2, 2] == 255 and np.all(np.isnan(back[2, 64:96]))
    fin = np.isfinite(back)
    # each block's largest element lands in [128, 256) before rounding: every element at or
    # above 2^-6 of the scale is a normal E4M3 value, off by at most 2^-4 relative
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    normal = fin & (np.abs(x) >= s * 2.0 ** -6)
    assert np.all(np.abs(back[normal] - x[normal]) <= np.abs(x[normal]) * 2.0 ** -4)
    small = fin & ~normal
    assert np.all(np.abs(back[small] - x[small]) <= s[small] * 2.0 ** -10)
