"""Pins of the oracle's T16 decoder against facts fixed outside the oracle.

- hand-derived state values and a hand-derived stream (tests/golden);
- the closed form of the byte-sum distribution over all 65,536 states;
- the bitshift-trellis overlap and round-trip properties at every position, wrap included;
- an independent big-integer window decoder written here;
- the tile placement (column-major positions) via single-bit streams;
- the unit sizes printed in the exlr8 "Stores" table.
"""

import numpy as np
import pytest

import oracle
from workloads import random_words, rng_for


def _hex(s):
    return int(s, 16)


def test_spot_values(golden):
    for state, prod, bsum, q in golden("t16_states.txt"):
        s = _hex(state)
        assert (s * oracle.T16_MULT) % 65536 == _hex(prod)
        assert oracle.t16_value(s) == int(q)
        assert int(q) == int(bsum) - 255


def test_exhaustive_distribution():
    # 0x3A2F is odd, so s -> s*0x3A2F mod 2^16 is a bijection: (low, high) take every
    # byte pair once and low + high has the triangular histogram min(v+1, 511-v),
    # mean 255 and variance 2 * (256^2 - 1) / 12 = 10922.5.
    q = oracle.t16_value_array(np.arange(65536))
    assert q.min() == -255 and q.max() == 255
    hist = np.bincount(q + 255, minlength=511)
    v = np.arange(511)
    assert np.array_equal(hist, np.minimum(v + 1, 511 - v))
    assert q.mean() == 0.0
    assert np.isclose(q.astype(np.float64).var(), 10922.5, rtol=0, atol=1e-9)
    m = (np.arange(65536) * oracle.T16_MULT) % 65536
    assert np.unique(m).size == 65536


def test_scalar_and_array_values_agree():
    s = np.arange(0, 65536, 7)
    assert [oracle.t16_value(int(v)) for v in s] == list(oracle.t16_value_array(s))


def _example_words(K):
    return [(0x9E3779B9 * (j + 1)) % (1 << 32) for j in range(8 * K)]


def test_stream_example(golden):
    for K, p, state, q in golden("trellis_stream_example.txt"):
        K, p = int(K), int(p)
        states = oracle.tile_states_scalar(_example_words(K), K)
        assert states[p] == _hex(state), (K, p)
        if q != "x":
            assert oracle.t16_value(states[p]) == int(q)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_overlap_and_round_trip(K):
    rng = rng_for(100, 0, K)
    for _ in range(4):
        words = [int(w) for w in random_words(rng, 8 * K)]
        states = oracle.tile_states_scalar(words, K)
        bits = oracle.tile_bits_scalar(words, K)
        n = 256 * K
        mask = (1 << (16 - K)) - 1
        for p in range(256):
            nxt = states[(p + 1) % 256]
            # bitshift trellis: the next window drops the first K bits of this one
            assert nxt >> K == states[p] & mask
            # the top K bits of state p are stream bits pK .. pK+K-1 (round trip)
            top = states[p] >> (16 - K)
            expect = 0
            for j in range(K):
                expect = expect * 2 + bits[(p * K + j) % n]
            assert top == expect
        # every bit lies in floor(16/K) or ceil(16/K) windows
        cover = np.zeros(n, dtype=np.int64)
        for p in range(256):
            for j in range(16):
                cover[(p * K + j) % n] += 1
        assert set(np.unique(cover)) <= {16 // K, -(-16 // K)}


def _bigint_states(words, K):
    """Independent decoder: the tile as one big integer, windows cut by rotation."""
    n = 32 * len(words)
    big = 0
    for w in words:
        big = (big << 32) | int(w)
    out = []
    for p in range(256):
        start = p * K
        rot = ((big << start) | (big >> (n - start))) & ((1 << n) - 1) if start else big
        out.append(rot >> (n - 16))
    return out


@pytest.mark.parametrize("K", [2, 3, 4])
def test_independent_bigint_decoder(K):
    rng = rng_for(100, 1, K)
    for _ in range(8):
        words = [int(w) for w in random_words(rng, 8 * K)]
        assert oracle.tile_states_scalar(words, K) == _bigint_states(words, K)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("shape", [(16, 16), (32, 48), (48, 32)])
def test_scalar_vs_vectorised_unit(K, shape):
    out, inputs = shape
    words = random_words(rng_for(100, 2, K, out, inputs), out * inputs * K // 32)
    q_vec = oracle.decode_unit(words, K, out, inputs)
    q_sc = np.array(oracle.decode_unit_scalar(words, K, out, inputs))
    assert q_vec.shape == (out, inputs)
    assert np.array_equal(q_vec, q_sc)


def test_single_bit_placement():
    # One set bit at stream position 0 of tile (to=1, ti=2) of a 32 x 48 unit (K=2).
    # Windows containing bit 0: p = 0 (offset 0) and, through the wrap, p = 249..255.
    # Column-major positions put p at (output 16*to + p//16, input 16*ti + p%16).
    K, out, inputs = 2, 32, 48
    n_ti = inputs // 16
    words = np.zeros(out * inputs * K // 32, dtype=np.uint32)
    tile = 1 * n_ti + 2
    words[tile * 8 * K] = 0x80000000
    q = oracle.decode_unit(words, K, out, inputs)
    base = oracle.t16_value(0)
    hot = {(int(o), int(i)) for o, i in zip(*np.nonzero(q != base))}
    expect = {(16 + 0, 32 + 0)} | {(16 + 15, 32 + p - 240) for p in range(249, 256)}
    assert hot == expect
    states = oracle.tile_states_scalar([int(w) for w in words[tile * 16:(tile + 1) * 16]], K)
    assert states[0] == 0x8000
    assert [states[p] for p in range(249, 256)] == [1 << (15 - (256 * K - p * K)) for p in range(249, 256)]


def test_all_zero_and_all_one_streams():
    z = oracle.decode_unit(np.zeros(16, dtype=np.uint32), 2, 16, 16)
    assert np.all(z == oracle.t16_value(0))
    o = oracle.decode_unit(np.full(16, 0xFFFFFFFF, dtype=np.uint32), 2, 16, 16)
    assert np.all(o == oracle.t16_value(0xFFFF))


def test_unit_sizes(golden):
    sizes = {row[0]: row[1] for row in golden("store_sizes.txt")}
    for K in (2, 3, 4):
        assert oracle.unit_bytes(K) == int(sizes["k%d" % K])
        assert oracle.unit_bytes(K) / (128 * 5120) == K / 8  # 0.25 / 0.375 / 0.5 B per weight
