"""Pins of the oracle's routed contraction and route bucketing: exact-rational brute force,
one-hot inputs, gate linearity, empty / invalid slots, and a brute-force stable sort."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import bf16_from_normal, fp16_scales, random_words, rng_for


def _layer(seed, E, out, inputs, K):
    words = [random_words(rng_for(103, seed, e), out * inputs * K // 32) for e in range(E)]
    q = [oracle.decode_unit(w, K, out, inputs) for w in words]
    sc = oracle.f16_bits_to_f64(fp16_scales(rng_for(103, seed + 50), (E, out), inputs))
    return q, sc


@pytest.mark.parametrize("shape,K", [((16, 16), 2), ((32, 32), 3), ((32, 32), 4), ((256, 256), 2)])
def test_fp64_matches_exact_rationals(shape, K):
    out, inputs = shape
    E, T, topk = (2, 3, 2) if out < 256 else (1, 1, 1)
    q, sc = _layer(1, E, out, inputs, K)
    x = bf16_from_normal(rng_for(103, 2, out), (T, inputs))
    ids = (np.arange(T * topk).reshape(T, topk) % E).astype(np.int32)
    gates = np.array([[0.25, 0.75], [1.0, 0.5], [0.125, 2.0]])[:T, :topk]
    y = oracle.expert_gemm(x, ids, gates, E, lambda e: q[e], lambda e: sc[e])
    exact = oracle.expert_gemm_exact(oracle.bf16_bits_to_f64(x), ids, gates, E, out,
                                     lambda e: q[e], lambda e: sc[e])
    for t in range(T):
        for k in range(topk):
            ref = np.array([float(v) for v in exact[t][k]])
            err = np.linalg.norm(y[t, k] - ref) / np.linalg.norm(ref)
            assert err <= 1e-12


def test_one_hot_selects_a_weight_column():
    q, sc = _layer(3, 1, 32, 48, 3)
    x = np.zeros((1, 48), dtype=np.uint16)
    x[0, 17] = 0x3F80  # 1.0
    y = oracle.expert_gemm(x, np.zeros((1, 1), np.int32), None, 1, lambda e: q[e], lambda e: sc[e])
    assert np.array_equal(y[0, 0], sc[0] * q[0][:, 17])


def test_gate_linearity_empty_and_invalid_slots():
    q, sc = _layer(4, 3, 16, 32, 2)
    x = bf16_from_normal(rng_for(103, 5), (2, 32))
    ids = np.array([[0, -1, 2], [5, 1, -3]], dtype=np.int32)
    g1 = np.ones((2, 3))
    g2 = np.full((2, 3), 0.5)
    y1 = oracle.expert_gemm(x, ids, g1, 3, lambda e: q[e], lambda e: sc[e])
    y2 = oracle.expert_gemm(x, ids, g2, 3, lambda e: q[e], lambda e: sc[e])
    assert np.array_equal(y2[0, 0], 0.5 * y1[0, 0])
    assert np.all(y1[0, 1] == 0)
    assert np.all(np.isnan(y1[1, 0])) and np.all(np.isnan(y1[1, 2]))
    comb = oracle.combine_slots(np.nan_to_num(y1))
    assert np.allclose(comb[0], y1[0, 0] + y1[0, 2])


def test_route_bucket_against_sorted():
    rng = rng_for(103, 6)
    E = 37
    ids = rng.integers(-2, E + 2, size=(50, 6)).astype(np.int32)
    counts, offsets, pairs, empty, invalid = oracle.route_bucket(ids, E)
    flat = ids.reshape(-1)
    valid = [(int(e), i) for i, e in enumerate(flat) if 0 <= e < E]
    assert list(pairs) == [i for _, i in sorted(valid)]
    assert list(counts) == [sum(1 for v in flat if v == e) for e in range(E)]
    assert offsets[0] == 0 and list(np.diff(offsets)) == list(counts)
    assert list(empty) == [i for i, e in enumerate(flat) if e == -1]
    assert list(invalid) == [i for i, e in enumerate(flat) if e < -1 or e >= E]
