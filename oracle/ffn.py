"""Routed expert FFN: the fused gate/up projection, SwiGLU, the rotated down projection, the
gate-weighted combine (FORMAT F15), with optional output-side rotations (F17).

Source passages: DeepSeek-V4.1-Flash-1017 · exlr8 page, "Layout" and "Stores" (every expert
projection is cut into units of 128 intermediate channels; gate and up stored together;
trellis units carry 128 x 128 Hadamard rotations on both sides); DeepSeek-V4.1-Flash-1017 ·
dsx T16 page, "October 25 runtime checkpoint" (fused gate/up post-processing, i.e. the gated
activation applied to the two projections).

TEST INFRASTRUCTURE (see the package docstring). Every step is FP64; the intermediate is
neither rounded nor quantised (the GPU's operand conversions are covered by the parity
bound).
"""

import math

import numpy as np

from .gemm import expert_gemm, expert_gemm_values
from .hadamard import output_rotation128, rotate128_values


def silu(a):
    """a / (1 + e^-a), elementwise, FP64 (stable for large |a|)."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    e = np.exp(a[~pos])
    out[~pos] = a[~pos] * e / (1.0 + e)
    return out


def silu_scalar(a):
    """The same function for one Python float, written directly from its definition."""
    return a / (1.0 + math.exp(-a)) if a >= 0 else a * math.exp(a) / (1.0 + math.exp(a))


def expert_ffn(x_bits, topk_ids, topk_w, E, gate_up_fns, down_fns, down_signs,
               gate_up_out_signs=None, down_out_signs=None):
    """FP64 y [T, H] of the routed expert FFN.

    x_bits: bf16 patterns [T, H] of the (rotated) input. gate_up_fns, down_fns: (weight_of,
    scale_of) pairs as for expert_gemm (gate_up [2I, H]: the gate's I channels, then the
    up's; down [H, I]). down_signs: int8 [I] or None (the rotation of the intermediate).
    *_out_signs: the output-side rotation of a projection (F17), or None for none.
    topk_w: [T, topk] or None.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    gu = expert_gemm(x_bits, ids, None, E, *gate_up_fns)       # [T, topk, 2I]
    if gate_up_out_signs is not None:
        gu = output_rotation128(gu, gate_up_out_signs)
    I = gu.shape[2] // 2
    g, u = gu[:, :, :I], gu[:, :, I:]
    h = (silu(g) * u).reshape(T * topk, I)
    v = rotate128_values(h, down_signs)
    gates = None if topk_w is None else np.asarray(topk_w, dtype=np.float64).reshape(T * topk, 1)
    z = expert_gemm_values(v, ids.reshape(T * topk, 1), gates, E, *down_fns)  # [T*topk, 1, H]
    if down_out_signs is not None:
        z = output_rotation128(z, down_out_signs)
    z = z.reshape(T, topk, -1)
    y = np.zeros((T, z.shape[2]), dtype=np.float64)
    for k in range(topk):
        y = y + z[:, k, :]
    return y
