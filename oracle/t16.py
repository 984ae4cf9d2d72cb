"""T16 bitshift-trellis decoding, written from the definition (FORMAT F1-F5).

Source passages (DeepSeek-V4.1-Flash-1017 · dsx T16 page, section "How T16 works"):
- opening paragraph: the experts use a QTIP-style bitshift trellis;
- item 1: a weight comes from its 16-bit window of the bit stream, multiplied by the
  16-bit constant 0x3A2F, and the two bytes of the product are added;
- item 2: positions are column-major inside each 16 x 16 tile.
Unit sizes: DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores" table (k2/k3/k4 rows).

Two implementations:
- ``*_scalar``: pure-Python loops over an explicit list of bits (small cases);
- ``decode_unit``: the same steps vectorised with NumPy (unit-sized cases).
Both return the integer matrix q in HF orientation, q[out, in] (row = output channel).
"""

import numpy as np

T16_MULT = 0x3A2F
TILE = 16
POSITIONS = TILE * TILE  # 256 trellis positions per tile


def unit_bytes(K, out=128, inputs=5120):
    """Bytes of one trellis unit: K bits per weight, no side data (FORMAT F2)."""
    assert (out * inputs * K) % 8 == 0
    return out * inputs * K // 8


def t16_value(state):
    """q for one 16-bit state (FORMAT F5; T16 page item 1).

    The product is taken modulo 2^16 (a 16-bit multiply); its low and high bytes are
    unsigned and added; 255, the exact mean of that sum, is subtracted.
    """
    if not 0 <= state < 65536:
        raise ValueError("state must be a 16-bit value")
    m = (state * T16_MULT) % 65536
    low = m % 256
    high = m // 256
    return low + high - 255


def t16_value_array(states):
    """Vectorised ``t16_value`` over an integer array of 16-bit states."""
    s = np.asarray(states, dtype=np.int64)
    if s.size and (s.min() < 0 or s.max() > 65535):
        raise ValueError("states must be 16-bit values")
    m = (s * T16_MULT) % 65536
    return (m % 256) + (m // 256) - 255


# ----------------------------------------------------------------------------------
# scalar path: explicit bit lists
# ----------------------------------------------------------------------------------

def tile_bits_scalar(words, K):
    """The tile's bit stream as a list of 0/1, most significant bit of word 0 first
    (FORMAT F3). A tile holds 256 positions x K bits = 8K words."""
    if len(words) != 8 * K:
        raise ValueError("a tile has 8*K words")
    bits = []
    for w in words:
        w = int(w)
        for b in range(31, -1, -1):
            bits.append((w >> b) & 1)
    return bits


def tile_states_scalar(words, K):
    """The 256 states of a tile: state p is the 16-bit window starting at bit p*K,
    read circularly (FORMAT F4: tail-biting inside the tile)."""
    bits = tile_bits_scalar(words, K)
    n = len(bits)
    states = []
    for p in range(POSITIONS):
        s = 0
        for j in range(16):
            s = s * 2 + bits[(p * K + j) % n]
        states.append(s)
    return states


def decode_tile_scalar(words, K):
    """q of one tile as a 16x16 list indexed [out_local][in_local]: position p holds
    input p mod 16 of output channel p // 16 (FORMAT F1; T16 page item 2)."""
    states = tile_states_scalar(words, K)
    q = [[0] * TILE for _ in range(TILE)]
    for p, s in enumerate(states):
        q[p // TILE][p % TILE] = t16_value(s)
    return q


def decode_unit_scalar(words, K, out, inputs):
    """q[out][inputs] of a whole unit from its uint32 words, tiles in strip-major
    order (FORMAT F2). Pure Python; meant for small matrices."""
    if out % TILE or inputs % TILE:
        raise ValueError("out and inputs must be multiples of 16")
    n_ti = inputs // TILE
    tw = 8 * K
    words = [int(w) for w in np.asarray(words, dtype=np.uint32).reshape(-1)]
    if len(words) != (out // TILE) * n_ti * tw:
        raise ValueError("word count does not match the unit shape")
    q = [[0] * inputs for _ in range(out)]
    for to in range(out // TILE):
        for ti in range(n_ti):
            t = to * n_ti + ti
            tq = decode_tile_scalar(words[t * tw:(t + 1) * tw], K)
            for ol in range(TILE):
                for il in range(TILE):
                    q[TILE * to + ol][TILE * ti + il] = tq[ol][il]
    return q


# ----------------------------------------------------------------------------------
# vectorised path: the same steps on arrays
# ----------------------------------------------------------------------------------

def _window_index(K):
    """idx[p, j] = (p*K + j) mod 256K: the stream bit feeding bit j of state p."""
    p = np.arange(POSITIONS)[:, None]
    j = np.arange(16)[None, :]
    return (p * K + j) % (POSITIONS * K)


def decode_unit(words, K, out, inputs):
    """Vectorised ``decode_unit_scalar``: returns q as an int16 array [out, inputs]."""
    if K not in (2, 3, 4):
        raise ValueError("K must be 2, 3 or 4")
    if out % TILE or inputs % TILE:
        raise ValueError("out and inputs must be multiples of 16")
    n_to, n_ti = out // TILE, inputs // TILE
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    if w.size != n_to * n_ti * 8 * K:
        raise ValueError("word count does not match the unit shape")
    # Bits, MSB first per word: write each word big-endian, then unpack bytes MSB first.
    bits = np.unpackbits(w.astype(">u4").view(np.uint8)).reshape(n_to * n_ti, 256 * K)
    win = bits[:, _window_index(K)]                           # [tiles, 256, 16], MSB first
    two = np.packbits(win, axis=-1).astype(np.int64)          # the window as 2 bytes
    states = two[..., 0] * 256 + two[..., 1]                  # [tiles, 256]
    qt = t16_value_array(states).reshape(n_to, n_ti, TILE, TILE)  # [to, ti, o_l, i_l]
    q = qt.transpose(0, 2, 1, 3).reshape(out, inputs)
    return q.astype(np.int16)


def decode_units128(words, K, out, inputs):
    """q [out, inputs] of a projection stored as inputs/128 units of 128 input channels
    (FORMAT F2b; exlr8 page, "Layout": units of 128 intermediate channels, the inputs of the
    down projection): unit j is an out x 128 strip-major unit (F2) holding inputs
    128 j .. 128 j + 127, units back to back."""
    if inputs % 128:
        raise ValueError("inputs must be a multiple of 128")
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    per = out * 128 * K // 32
    if w.size != per * (inputs // 128):
        raise ValueError("word count does not match the unit shape")
    return np.concatenate([decode_unit(w[j * per:(j + 1) * per], K, out, 128)
                           for j in range(inputs // 128)], axis=1)
