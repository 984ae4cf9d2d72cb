"""Route bucketing: group the (token, slot) pairs of a top-k routing by expert.

The pages do not describe the dispatch; they state that layers are routed and that
route kernels replay under graphs with changing routes (DeepSeek-V4.1-Flash-1017 TrellisMX
K2 Mix page, intro). The plainest reading (FORMAT F11, F14): a stable counting sort of the
flat slot indices t * topk + k by expert id. Slots with id -1 are empty; ids outside
[-1, E) are invalid.
"""

import numpy as np


def route_bucket(topk_ids, E):
    """Returns (counts [E], offsets [E+1], pairs, empty, invalid).

    pairs lists the flat indices of valid slots ordered by (expert, flat index);
    offsets[e] .. offsets[e+1] is expert e's range in it. empty / invalid list the flat
    indices of slots with id -1 / with an id outside [-1, E), ascending.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in ids:
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    pairs = np.zeros(int(offsets[-1]), dtype=np.int64)
    empty, invalid = [], []
    for i, e in enumerate(ids):           # ascending i keeps each bucket stable
        if 0 <= e < E:
            pairs[cursor[e]] = i
            cursor[e] += 1
        elif e == -1:
            empty.append(i)
        else:
            invalid.append(i)
    return counts, offsets, pairs, np.array(empty, dtype=np.int64), np.array(invalid, dtype=np.int64)
