"""GPU hadamard128 and route_bucket vs the oracle, bit for bit."""

import numpy as np
import pytest

import oracle
from gpu_helpers import dev, gpu, needs_gpu, ops, to_dev, torch
from workloads import bf16_from_normal, random_signs, rng_for, uniform_routes, zipf_routes

pytestmark = [gpu, needs_gpu]


@pytest.mark.parametrize("rows,n,with_signs", [(1, 128, False), (37, 5120, True), (3, 256, True),
                                               (1025, 1024, False)])
def test_hadamard_bit_exact(rows, n, with_signs):
    x = bf16_from_normal(rng_for(300, rows, n), (rows, n))
    s = random_signs(rng_for(301, n), n) if with_signs else None
    y = ops().hadamard128(to_dev(x, np.int16), None if s is None else to_dev(s))
    ref = oracle.hadamard128_fp32_order(x, s)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), ref)


def test_hadamard_in_place_and_extremes():
    x = bf16_from_normal(rng_for(302, 0), (4, 512))
    x[0, :] = np.uint16(0x7F7F)           # bf16 max: sums overflow to inf
    x[1, 5] = np.uint16(0x7FC0)           # NaN poisons its block
    x[2, :128] = np.uint16(0x0001)        # subnormals
    s = random_signs(rng_for(302, 1), 512)
    xd = to_dev(x, np.int16)
    ops().hadamard128(xd, to_dev(s), out=xd)
    got = xd.cpu().numpy().view(np.uint16)
    ref = oracle.hadamard128_fp32_order(x, s)
    gv, rv = oracle.bf16_bits_to_f64(got), oracle.bf16_bits_to_f64(ref)
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    fin = ~np.isnan(rv)
    assert np.array_equal(got[fin], ref[fin])


def _route_case(ids, E):
    counts, offsets, pairs = ops().route_bucket(to_dev(ids), E)
    c, o, p, _, _ = oracle.route_bucket(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(pairs.cpu().numpy()[:o[-1]], p)


def test_route_uniform_decode_batch():
    _route_case(uniform_routes(rng_for(303, 0), 128, 384, 8), 384)


def test_route_zipf_prefill_chunk():
    _route_case(zipf_routes(rng_for(303, 1), 8192, 384, 8), 384)


def test_route_ragged_empty_and_invalid():
    rng = rng_for(303, 2)
    ids = rng.integers(-3, 70, size=(333, 5)).astype(np.int32)  # -1 empty, others invalid
    _route_case(ids, 64)
    _route_case(np.full((7, 3), -1, np.int32), 16)
    _route_case(rng.integers(0, 1, size=(2049, 1)).astype(np.int32), 1)
    _route_case(rng.integers(0, 4096, size=(3000, 2)).astype(np.int32), 4096)


def test_route_is_deterministic():
    ids = to_dev(zipf_routes(rng_for(303, 3), 4096, 384, 8))
    a = [t.cpu().numpy() for t in ops().route_bucket(ids, 384)]
    b = [t.cpu().numpy() for t in ops().route_bucket(ids, 384)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
