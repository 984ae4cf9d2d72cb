"""Tail-biting Viterbi encoder for bitshift-trellis codes (T16 and the other codebooks).

TEST INFRASTRUCTURE (see the package docstring): it produces code streams for the decode
round trip and measures the distortion the codebooks reach; it is not on the product path.

Source passages: DeepSeek-V4.1-Flash-1017 · dsx T16 page, "How T16 works" (opening
paragraph: the bitshift trellis is found by a Viterbi search; item 1: T16 has about 4 %
more error than exllamav3's codebook on random data). The stream structure is FORMAT F1-F4:
a tile of P positions is a circular stream of P K bits and position p takes the L-bit
window at bit p K (L = 16 for T16 and mul1).

The search. Consecutive windows overlap: s_{p+1} = ((s_p << K) mod 2^L) | (K new bits), so
the predecessors of a state s' are the 2^K states whose low L - K bits equal s' >> K. The
stream is circular, so a valid state sequence also satisfies
  (top L - K bits of s_0) = (low L - K bits of s_{P-1}).
Given the value c of those shared bits, the cheapest valid sequence is a Viterbi search
whose first state is restricted to the 2^K states with top bits c and whose last state to
those with low bits c. The exact tail-biting optimum is the best over all 2^(L - K) values
of c (``encode_tile(..., exact=True)``, practical for small L). For L = 16 the encoder
descends over two cuts of the circle (positions 0 and P / 2): an unconstrained search with
its ends at the second cut gives the bits that cross the first; each round then ties one
cut to the bits the current path crosses it with and searches again. Every round returns a
valid tail-biting stream at no higher cost than the last, and the result is optimal
whenever the optimum crosses a cut with the bits tried there.

Cost: squared error, sum_p (w_p - scale * value[s_p])^2.
"""

import numpy as np


def _search(err, K, L, first_top=None, last_low=None):
    """Cheapest state path through the per-position cost rows err [P, 2^L]: returns
    (cost, states [P]). first_top / last_low restrict the first state's top L - K bits and
    the last state's low L - K bits (None: free)."""
    P, n = err.shape
    low_bits = L - K
    inf = np.inf
    cost = err[0].copy()
    if first_top is not None:
        allowed = (np.arange(n) >> K) == first_top
        cost[~allowed] = inf
    back = np.zeros((P, n), dtype=np.uint16 if K > 8 else np.uint8)
    succ_low = np.arange(n) >> K                 # low L - K bits of each state's predecessors
    for p in range(1, P):
        by_top = cost.reshape(1 << K, 1 << low_bits)  # [top K bits, low L - K bits]
        top = np.argmin(by_top, axis=0)
        best = by_top[top, np.arange(1 << low_bits)]
        cost = err[p] + best[succ_low]
        back[p] = top[succ_low]
    if last_low is not None:
        ok = (np.arange(n) & ((1 << low_bits) - 1)) == last_low
        cost = np.where(ok, cost, inf)
    s = int(np.argmin(cost))
    total = float(cost[s])
    states = np.zeros(P, dtype=np.int64)
    states[P - 1] = s
    for p in range(P - 1, 0, -1):
        prev = (int(back[p][s]) << low_bits) | (s >> K)
        states[p - 1] = prev
        s = prev
    return total, states


def _cut_search(err, K, L, a, c):
    """The cheapest circular path whose states at positions a - 1 and a share the bits c
    (the stream cut between them): the search over positions a, a + 1, ... (circularly)
    with both ends tied to c. Returns (cost, states in original position order)."""
    P = err.shape[0]
    order = (np.arange(P) + a) % P
    total, st = _search(err[order], K, L, first_top=c, last_low=c)
    states = np.empty(P, dtype=np.int64)
    states[order] = st
    return total, states


def _descend(err, K, L, rounds=6):
    """Circular path by alternating cuts (0 and P / 2): the first cut's bits come from an
    unconstrained search across it; then each round ties the other cut to the bits the
    current path crosses it with. Every round's path is a valid circular stream and costs
    no more than the last (the last path is feasible for the new search)."""
    P = err.shape[0]
    low = (1 << (L - K)) - 1
    h = P // 2
    _, st = _cut_search(err, K, L, h, None)     # free ends at cut h: cut 0 is interior
    cut = 0
    best_total, best = np.inf, None
    for _ in range(rounds):
        c = int(st[(cut - 1) % P]) & low
        total, st = _cut_search(err, K, L, cut, c)
        if total >= best_total - 1e-12 * max(1.0, best_total):
            break
        best_total, best = total, st
        cut = h if cut == 0 else 0
    return best_total, best


def _cost_rows(w, values, scale):
    w = np.asarray(w, dtype=np.float64).reshape(-1, 1)
    return (w - scale * np.asarray(values, dtype=np.float64)[None, :]) ** 2


def encode_tile(w, K, values, scale=1.0, L=16, exact=False):
    """Tail-biting encode of one tile's weights w [P] (position order) with the codebook
    `values` [2^L]. Returns (bits [P K] as 0/1, states [P], squared error)."""
    err = _cost_rows(w, values, scale)
    P = err.shape[0]
    if P * K < L:
        raise ValueError("the stream must be at least one window long")
    low_bits = L - K
    if exact:
        best = (np.inf, None)
        for c in range(1 << low_bits):
            tot, st = _search(err, K, L, first_top=c, last_low=c)
            if tot < best[0]:
                best = (tot, st)
        total, states = best
    else:
        total, states = _descend(err, K, L)
    bits = np.zeros(P * K, dtype=np.uint8)
    for p in range(P):
        own = int(states[p]) >> low_bits                   # the state's first K bits
        for j in range(K):
            bits[p * K + j] = (own >> (K - 1 - j)) & 1
    return bits, states, total


def stream_states(bits, K, L=16):
    """The states of a circular stream (the decoder's view, FORMAT F4): window at p K."""
    bits = np.asarray(bits, dtype=np.int64)
    n = bits.size
    P = n // K
    idx = (np.arange(P)[:, None] * K + np.arange(L)[None, :]) % n
    return (bits[idx] * (1 << np.arange(L - 1, -1, -1))[None, :]).sum(axis=1)


def bits_to_words(bits):
    """MSB-first packing of a stream into uint32 words (FORMAT F3)."""
    b = np.asarray(bits, dtype=np.uint8).reshape(-1, 32)
    return (b.astype(np.uint64) << np.arange(31, -1, -1, dtype=np.uint64)).sum(axis=1).astype(np.uint32)


def encode_unit(W, K, values, scale=1.0):
    """Encode a weight matrix W [out, in] (HF orientation, multiples of 16) tile by tile
    into a strip-major unit (FORMAT F2) with codebook `values` [65536]. Returns
    (uint32 words, reconstruction [out, in] = scale * value of each chosen state, total
    squared error)."""
    W = np.asarray(W, dtype=np.float64)
    out, inp = W.shape
    n_to, n_ti = out // 16, inp // 16
    words = []
    recon = np.zeros_like(W)
    total = 0.0
    for to in range(n_to):
        for ti in range(n_ti):
            tile = W[16 * to:16 * to + 16, 16 * ti:16 * ti + 16]   # [o_l, i_l]
            w = tile.reshape(-1)                                  # position p = 16 o_l + i_l
            bits, states, err = encode_tile(w, K, values, scale)
            words.append(bits_to_words(bits))
            recon[16 * to:16 * to + 16, 16 * ti:16 * ti + 16] = \
                (scale * np.asarray(values)[states]).reshape(16, 16)
            total += err
    return np.concatenate(words), recon, total
