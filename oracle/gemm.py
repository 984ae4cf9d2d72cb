"""Routed-expert contraction: y[t, k, o] = g[t, k] * scale_e[o] * sum_i x[t, i] * W_e[o, i].

Source passages: DeepSeek-V4.1-Flash-1017 · dsx T16 page, "How T16 works" item 4 (the
stored per-output scale multiplies each output channel); the unit shape of the
DeepSeek-V4.1-Flash-1017 · exlr8 page, "Layout"; FORMAT F6, F10, F11.

W_e is the decoded weight matrix in HF orientation [out, in]: the integer q of a trellis
expert, or the exact MXFP4 values. The contraction is FP64 over exactly the bf16 input
values the GPU consumes; a library matmul is the summation step. ``expert_gemm_exact`` is
the same definition in exact rational arithmetic, for brute-force checks.
"""

from fractions import Fraction

import numpy as np

from .fpbits import bf16_bits_to_f64


def expert_gemm(x_bits, topk_ids, topk_w, E, weight_of, scale_of=None):
    """FP64 per-slot outputs [T, topk, out].

    x_bits: bf16 patterns [T, in]. weight_of(e) -> float64 [out, in].
    scale_of(e) -> float64 [out] or None (scale 1). topk_w: [T, topk] or None (gate 1).
    Empty slots (-1) give 0; ids outside [-1, E) give NaN.
    """
    return expert_gemm_values(bf16_bits_to_f64(x_bits), topk_ids, topk_w, E, weight_of,
                              scale_of)


def expert_gemm_values(x_vals, topk_ids, topk_w, E, weight_of, scale_of=None):
    """``expert_gemm`` of activations given as FP64 values [T, in] (an intermediate that is
    not rounded to a storage format, FORMAT F15)."""
    x = np.asarray(x_vals, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    gates = None if topk_w is None else np.asarray(topk_w, dtype=np.float64)
    out = None
    y = None
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        if not 0 <= e < E:
            continue
        w = np.asarray(weight_of(e), dtype=np.float64)
        if y is None:
            out = w.shape[0]
            y = np.zeros((T, topk, out), dtype=np.float64)
        t_idx, k_idx = np.nonzero(ids == e)
        acc = x[t_idx] @ w.T                                   # [n, out]
        if scale_of is not None:
            acc = acc * np.asarray(scale_of(e), dtype=np.float64)[None, :]
        if gates is not None:
            acc = acc * gates[t_idx, k_idx][:, None]
        y[t_idx, k_idx] = acc
    if y is None:
        raise ValueError("no valid slot: output width unknown")
    bad = (ids < -1) | (ids >= E)
    y[bad] = np.nan
    return y


def expert_gemm_exact(x_vals, topk_ids, topk_w, E, out, weight_of, scale_of=None):
    """The same definition with Fractions: every input converted exactly, no rounding.

    x_vals are floats that are exact binary fractions (e.g. decoded bf16). weight_of(e)
    returns an [out][in] array of integers or exact floats. Returns nested lists
    [T][topk][out] of Fractions; an invalid slot holds None.
    """
    ids = [[int(v) for v in row] for row in np.asarray(topk_ids)]
    xs = [[Fraction(float(v)) for v in row] for row in np.asarray(x_vals, dtype=np.float64)]
    result = []
    for t, row in enumerate(ids):
        slots = []
        for k, e in enumerate(row):
            if e == -1:
                slots.append([Fraction(0)] * out)
                continue
            if not 0 <= e < E:
                slots.append(None)
                continue
            w = weight_of(e)
            sc = scale_of(e) if scale_of is not None else None
            g = Fraction(float(topk_w[t][k])) if topk_w is not None else Fraction(1)
            vals = []
            for o in range(out):
                acc = Fraction(0)
                for i, xv in enumerate(xs[t]):
                    acc += xv * Fraction(float(w[o][i]))
                s = Fraction(float(sc[o])) if sc is not None else Fraction(1)
                vals.append(g * s * acc)
            slots.append(vals)
        result.append(slots)
    return result


def combine_slots(y_slots):
    """y[t, o] = sum over k = 0 .. topk-1, in that order, of the per-slot outputs."""
    y = np.asarray(y_slots, dtype=np.float64)
    acc = np.zeros((y.shape[0], y.shape[2]), dtype=np.float64)
    for k in range(y.shape[1]):
        acc = acc + y[:, k, :]
    return acc
