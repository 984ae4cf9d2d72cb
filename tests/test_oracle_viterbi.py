"""Pins of the tail-biting Viterbi encoder (test infrastructure; dsx T16 page, "How T16
works": the bitshift trellis is found by a Viterbi search).

- optimality: on tiny circular streams (window L = 8 bits) the exact search equals brute
  force over every stream; the practical search (one guess of the wrap bits) is never
  better than the exact one and always returns a valid circular stream;
- validity at full size: the stream of a 256-position T16 tile decodes (oracle.decode_unit)
  to exactly the values the search chose;
- distortion: on Gaussian weights the squared error per weight is at least the
  rate-distortion bound 2^-2K and within 30 % of it (a search that did not optimise would
  land near the scalar quantiser's, e.g. 0.1175 at K = 2 against 0.0625).
"""

import numpy as np
import pytest

import oracle
from oracle import viterbi as vt
from workloads import rng_for


def _brute(w, K, values, L):
    P = w.size
    n = P * K
    streams = np.arange(1 << n, dtype=np.int64)
    bits = (streams[:, None] >> np.arange(n - 1, -1, -1)[None, :]) & 1     # [S, n], MSB first
    idx = (np.arange(P)[:, None] * K + np.arange(L)[None, :]) % n          # [P, L]
    states = (bits[:, idx] * (1 << np.arange(L - 1, -1, -1))).sum(axis=2)  # [S, P]
    cost = ((w[None, :] - values[states]) ** 2).sum(axis=1)
    return float(cost.min())


@pytest.mark.parametrize("K,P", [(2, 8), (3, 6), (4, 5), (2, 9)])
def test_exact_search_equals_brute_force(K, P):
    L = 8
    rng = rng_for(750, K, P)
    for trial in range(3):
        values = rng.standard_normal(1 << L)
        w = rng.standard_normal(P) * 1.3
        bits, states, err = vt.encode_tile(w, K, values, L=L, exact=True)
        assert abs(err - _brute(w, K, values, L)) <= 1e-9
        assert np.array_equal(vt.stream_states(bits, K, L), states)
        assert abs(((w - values[states]) ** 2).sum() - err) <= 1e-9
        _, pst, perr = vt.encode_tile(w, K, values, L=L, exact=False)
        assert perr >= err - 1e-9


def test_practical_search_valid_and_mostly_optimal():
    """Short circles with random value tables are the hard case for the cut descent (the
    wrap touches a large share of the positions): it must stay valid and never beat the
    exact search, and it finds the optimum in most trials (30 of 40 with these seeds,
    mean excess 3 %)."""
    L, K, P = 8, 2, 24
    rng = rng_for(751, 0)
    hits, gaps = 0, []
    for trial in range(40):
        values = rng.standard_normal(1 << L)
        w = rng.standard_normal(P)
        _, _, ex = vt.encode_tile(w, K, values, L=L, exact=True)
        bits, states, pr = vt.encode_tile(w, K, values, L=L)
        assert np.array_equal(vt.stream_states(bits, K, L), states)
        assert pr >= ex - 1e-9
        hits += pr <= ex + 1e-9
        gaps.append(pr / ex - 1)
    assert hits >= 28 and np.mean(gaps) <= 0.05


@pytest.mark.parametrize("K", [2, 3, 4])
def test_t16_tile_round_trip(K):
    values = oracle.t16_value_array(np.arange(65536)).astype(np.float64)
    w = rng_for(752, K).standard_normal(256) * 100
    bits, states, err = vt.encode_tile(w, K, values)
    words = vt.bits_to_words(bits)
    q = oracle.decode_unit(words, K, 16, 16)                 # [o_l, i_l]
    assert np.array_equal(q.reshape(-1), values[states].astype(np.int64))
    assert abs(((w - values[states]) ** 2).sum() - err) <= 1e-6 * err


@pytest.mark.parametrize("K", [2, 3, 4])
def test_gaussian_distortion_near_the_bound(K):
    values = oracle.t16_value_array(np.arange(65536)).astype(np.float64)
    rng = rng_for(753, K)
    W = rng.standard_normal((16, 64))                        # 4 tiles
    scale = {2: 0.9, 3: 1.2, 4: 1.25}[K] / values.std()
    words, recon, total = vt.encode_unit(W, K, values, scale)
    mse = total / W.size
    assert np.allclose(recon, scale * oracle.decode_unit(words, K, 16, 64))
    bound = 2.0 ** (-2 * K)
    print("K = %d: MSE %.5f, rate-distortion bound %.5f" % (K, mse, bound))
    assert bound <= mse <= 1.3 * bound
