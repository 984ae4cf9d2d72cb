"""Pins of the oracle's Hadamard rotation: the library Hadamard matrix, orthogonality,
involution, closed-form inputs, and the fp32-order form within one bf16 ulp of FP64."""

import numpy as np
import scipy.linalg

import oracle
from oracle.fpbits import f32_to_bf16_bits_rne
from workloads import bf16_from_normal, random_signs, rng_for


def test_matches_library_hadamard():
    assert np.array_equal(oracle.sylvester_hadamard(128), scipy.linalg.hadamard(128))


def test_orthogonal():
    h = oracle.sylvester_hadamard(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_f64_involution_and_norm():
    x = bf16_from_normal(rng_for(102, 3), (3, 256))
    y = oracle.hadamard128_f64(x)
    xv = oracle.bf16_bits_to_f64(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xv, axis=1), rtol=1e-13)
    h = scipy.linalg.hadamard(128) / np.sqrt(128.0)
    back = np.einsum("ij,rbj->rbi", h, y.reshape(3, 2, 128)).reshape(3, 256)
    assert np.allclose(back, xv, rtol=0, atol=1e-12)


def test_signs_apply_before_rotation():
    x = bf16_from_normal(rng_for(102, 4), (2, 128))
    s = random_signs(rng_for(102, 5), 128)
    h = scipy.linalg.hadamard(128) / np.sqrt(128.0)
    expect = (oracle.bf16_bits_to_f64(x) * s[None, :]) @ h.T
    assert np.allclose(oracle.hadamard128_f64(x, s), expect, rtol=0, atol=1e-12)


def test_one_hot_and_constant_inputs():
    one = np.uint16(0x3F80)                     # bf16 1.0
    x = np.zeros((2, 128), dtype=np.uint16)
    x[0, 5] = one
    x[1, :] = one
    y = oracle.hadamard128_fp32_order(x)
    # one-hot: column 5 of H / sqrt(128); fp32(1/sqrt 128) = 0x3DB504F3 rounds to bf16 0x3DB5
    col = scipy.linalg.hadamard(128)[:, 5]
    assert np.array_equal(y[0], np.where(col > 0, 0x3DB5, 0xBDB5).astype(np.uint16))
    # constant ones: H * 1 = 128 e_0, so y = sqrt(128) e_0
    expect1 = f32_to_bf16_bits_rne(np.float32(128.0) * np.uint32(0x3DB504F3).view(np.float32))
    assert y[1, 0] == expect1 and np.all(y[1, 1:] == 0)
    assert abs(oracle.bf16_bits_to_f64(y[1, 0]) - np.sqrt(128.0)) < 0.05


def test_fp32_order_within_one_bf16_ulp_of_f64():
    x = bf16_from_normal(rng_for(102, 6), (64, 512))
    s = random_signs(rng_for(102, 7), 512)
    emu = oracle.hadamard128_fp32_order(x, s).astype(np.int64)
    ref = f32_to_bf16_bits_rne(oracle.hadamard128_f64(x, s).astype(np.float32)).astype(np.int64)
    # same sign bits, magnitudes at most one bf16 ulp apart (adjacent patterns)
    assert np.array_equal(emu >> 15, ref >> 15)
    assert np.max(np.abs((emu & 0x7FFF) - (ref & 0x7FFF))) <= 1
    assert np.mean(emu == ref) > 0.95


def test_bf16_rounding_ties_to_even():
    v = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF], dtype=np.uint32).view(np.float32)
    assert list(f32_to_bf16_bits_rne(v)) == [0x3F80, 0x3F82, 0x3F81, 0x3F80]
