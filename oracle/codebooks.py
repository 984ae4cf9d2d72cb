"""The exlr8 trellis codebooks mul1 and pmcgx (FORMAT F20, F21), written from the page.

TEST INFRASTRUCTURE (see the package docstring).

Source passages: DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores" (the paragraph under the
table: each trellis file names its codebook, "pmcgx V2 L20 0xCBAC1FED/0xBCA14C51" or
"mul1 0x83DCD12D"; mul1 hashes one weight per state; pmcgx is a pair trellis in which two
weights share one 20-bit state, each weight the sum of the two fp16 halves of the state's
product with one of the two multipliers, rounded to FP8 E4M3); DeepSeek-V4.1-Flash-1017 ·
dsx T16 page, "How T16 works", item 1 (exllamav3's codebook spends a 32-bit multiply per
weight; T16 adds the bytes of a 16-bit product instead).

Both codebooks use the bitshift-trellis streams of FORMAT F1-F4 (16 x 16 tiles of 8K
little-endian words read MSB first, column-major positions, tail-biting per tile).

Readings where the page is silent (every one is "parity unpinned": the page prints no
decoded value and no file is available):
- mul1: the state is the 16-bit window of F4; m = state * 0x83DCD12D mod 2^32 and
  q = (sum of the four bytes of m) - 510, by analogy with T16's byte sum (510 is the exact
  mean of the sum of four uniform bytes), an integer in [-510, 510];
- pmcgx: pair j of a tile (positions 2j and 2j + 1, two consecutive inputs of one output
  channel) takes the 20-bit window that starts at stream bit 2Kj (tail-biting); with
  multiplier c_0 for position 2j and c_1 for 2j + 1, m = state * c mod 2^32, then
  x = (m & 0x8FFF8FFF) ^ 0x3B603B60 (the mask and xor of the published QTIP 3INST code,
  which keep each half a normal fp16 in [2^-3, 2)), the two halves of x read as fp16 are
  added exactly and the sum is rounded once to the nearest E4M3 value (ties to even).
"""

import numpy as np

from .fpbits import f16_bits_to_f64
from .mx import e4m3_all_values, e4m3_round
from .t16 import POSITIONS, TILE, _window_index, tile_bits_scalar, tile_states_scalar

MUL1_MULT = 0x83DCD12D
PMCGX_MULTS = (0xCBAC1FED, 0xBCA14C51)
PMCGX_MASK = 0x8FFF8FFF
PMCGX_XOR = 0x3B603B60
PMCGX_STATE_BITS = 20


# ---- mul1 ---------------------------------------------------------------------------------

def mul1_value(state):
    """q of one 16-bit state: the four bytes of state * 0x83DCD12D mod 2^32, added, minus
    510."""
    if not 0 <= state < 65536:
        raise ValueError("state must be a 16-bit value")
    m = (state * MUL1_MULT) % (1 << 32)
    return sum((m >> (8 * b)) & 0xFF for b in range(4)) - 510


def mul1_value_array(states):
    s = np.asarray(states, dtype=np.uint64)
    m = (s * np.uint64(MUL1_MULT)) & np.uint64(0xFFFFFFFF)
    total = np.zeros(s.shape, dtype=np.int64)
    for b in range(4):
        total += ((m >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.int64)
    return total - 510


def _unit_states16(words, K, out, inputs):
    """The 16-bit states of every position of a unit in strip-major tile order (F2):
    [out / 16, inputs / 16, 256]."""
    n_to, n_ti = out // TILE, inputs // TILE
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    if w.size != n_to * n_ti * 8 * K:
        raise ValueError("word count does not match the unit shape")
    bits = np.unpackbits(w.astype(">u4").view(np.uint8)).reshape(n_to * n_ti, 256 * K)
    two = np.packbits(bits[:, _window_index(K)], axis=-1).astype(np.int64)
    return (two[..., 0] * 256 + two[..., 1]).reshape(n_to, n_ti, POSITIONS)


def _to_matrix(per_tile, out, inputs):
    """[to, ti, 256] position values -> [out, inputs] (position p = 16 o_l + i_l)."""
    n_to, n_ti = out // TILE, inputs // TILE
    t = per_tile.reshape(n_to, n_ti, TILE, TILE)             # [to, ti, o_l, i_l]
    return t.transpose(0, 2, 1, 3).reshape(out, inputs)


def decode_unit_mul1(words, K, out, inputs):
    """q [out, inputs] (int16) of a mul1 unit."""
    if K not in (2, 3, 4):
        raise ValueError("K must be 2, 3 or 4")
    states = _unit_states16(words, K, out, inputs)
    return _to_matrix(mul1_value_array(states), out, inputs).astype(np.int16)


def decode_unit_mul1_scalar(words, K, out, inputs):
    """Pure-Python mul1 decode over explicit tile bit lists (small units)."""
    n_ti = inputs // TILE
    tw = 8 * K
    words = [int(v) for v in np.asarray(words, dtype=np.uint32).reshape(-1)]
    q = [[0] * inputs for _ in range(out)]
    for to in range(out // TILE):
        for ti in range(n_ti):
            base = (to * n_ti + ti) * tw
            states = tile_states_scalar(words[base:base + tw], K)
            for p, s in enumerate(states):
                q[TILE * to + p // TILE][TILE * ti + p % TILE] = mul1_value(s)
    return q


# ---- pmcgx --------------------------------------------------------------------------------

def pmcgx_half_sum(state, mult):
    """The exact sum of the two fp16 halves of (state * mult mod 2^32) after the mask and
    xor (FORMAT F21), as a Python float (exact: both halves lie in [2^-3, 2) in magnitude)."""
    m = (state * mult) % (1 << 32)
    x = (m & PMCGX_MASK) ^ PMCGX_XOR
    lo = float(f16_bits_to_f64(np.array([x & 0xFFFF], dtype=np.uint16))[0])
    hi = float(f16_bits_to_f64(np.array([x >> 16], dtype=np.uint16))[0])
    return lo + hi


def pmcgx_pair_codes(state):
    """E4M3 codes (first, second weight) of one 20-bit pair state."""
    if not 0 <= state < (1 << PMCGX_STATE_BITS):
        raise ValueError("state must be a 20-bit value")
    vals = [pmcgx_half_sum(state, c) for c in PMCGX_MULTS]
    return tuple(int(c) for c in e4m3_round(np.array(vals)))


def _pair_window_index(K):
    """idx[j, b] = (2Kj + b) mod 256K: the stream bit feeding bit b of pair state j."""
    j = np.arange(POSITIONS // 2)[:, None]
    b = np.arange(PMCGX_STATE_BITS)[None, :]
    return (2 * K * j + b) % (POSITIONS * K)


def _pmcgx_codes_of_states(states):
    s = np.asarray(states, dtype=np.uint64)
    out = []
    for c in PMCGX_MULTS:
        m = (s * np.uint64(c)) & np.uint64(0xFFFFFFFF)
        x = (m & np.uint64(PMCGX_MASK)) ^ np.uint64(PMCGX_XOR)
        lo = f16_bits_to_f64((x & np.uint64(0xFFFF)).astype(np.uint16))
        hi = f16_bits_to_f64((x >> np.uint64(16)).astype(np.uint16))
        out.append(e4m3_round(lo + hi))
    return out


def decode_unit_pmcgx(words, K, out, inputs):
    """E4M3 codes [out, inputs] (uint8) of a pmcgx unit."""
    if K not in (2, 3, 4):
        raise ValueError("K must be 2, 3 or 4")
    if out % TILE or inputs % TILE:
        raise ValueError("out and inputs must be multiples of 16")
    n_to, n_ti = out // TILE, inputs // TILE
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    if w.size != n_to * n_ti * 8 * K:
        raise ValueError("word count does not match the unit shape")
    bits = np.unpackbits(w.astype(">u4").view(np.uint8)).reshape(n_to * n_ti, 256 * K)
    win = bits[:, _pair_window_index(K)]                       # [tiles, 128, 20], MSB first
    weights = (1 << np.arange(PMCGX_STATE_BITS - 1, -1, -1)).astype(np.int64)
    states = win.astype(np.int64) @ weights                    # [tiles, 128]
    first, second = _pmcgx_codes_of_states(states)
    per_tile = np.stack([first, second], axis=-1).reshape(n_to, n_ti, POSITIONS)
    return _to_matrix(per_tile, out, inputs).astype(np.uint8)


def decode_unit_pmcgx_scalar(words, K, out, inputs):
    """Pure-Python pmcgx decode over explicit tile bit lists (small units)."""
    n_ti = inputs // TILE
    tw = 8 * K
    words = [int(v) for v in np.asarray(words, dtype=np.uint32).reshape(-1)]
    codes = [[0] * inputs for _ in range(out)]
    nbits = POSITIONS * K
    for to in range(out // TILE):
        for ti in range(n_ti):
            base = (to * n_ti + ti) * tw
            bits = tile_bits_scalar(words[base:base + tw], K)
            for j in range(POSITIONS // 2):
                s = 0
                for b in range(PMCGX_STATE_BITS):
                    s = 2 * s + bits[(2 * K * j + b) % nbits]
                for h, c in enumerate(pmcgx_pair_codes(s)):
                    p = 2 * j + h
                    codes[TILE * to + p // TILE][TILE * ti + p % TILE] = c
    return codes


def pmcgx_values(codes):
    """Values of E4M3 codes (the pmcgx weights before the channel scale)."""
    return e4m3_all_values()[np.asarray(codes, dtype=np.uint8)]


# ---- operands of the FP8 prefill ----------------------------------------------------------

def mul1_e4m3(q):
    """FORMAT F20's FP8 operand of mul1 values: 2 E4M3(q / 2) (q / 2 lies within E4M3's
    range; halving is exact), as float64."""
    q = np.asarray(q)
    if np.any(np.abs(q) > 510):
        raise ValueError("mul1 values lie in [-510, 510]")
    return 2.0 * e4m3_all_values()[e4m3_round(q.astype(np.float64) / 2.0)]
