"""Routed expert FFN: gate and up projections, SwiGLU, the rotated down projection, the
gate-weighted combine (FORMAT F15).

Source passages: DeepSeek-V4.1-Flash-1017 · exlr8 page, "Layout" and "Stores" (every expert
projection is cut into units of 128 intermediate channels; trellis units carry the 128-wide
Hadamard rotation); DeepSeek-V4.1-Flash-1017 · dsx T16 page, "October 25 runtime checkpoint"
(fused gate/up post-processing, i.e. the gated activation applied to the two projections).

TEST INFRASTRUCTURE (see the package docstring). Every step is FP64 except the two roundings
the definition fixes: the intermediate is rounded to bf16 (the operand precision of the down
projection) and rotated with the fp32-order rotation of FORMAT F8.
"""

import math

import numpy as np

from .fpbits import f32_to_bf16_bits_rne
from .gemm import expert_gemm
from .hadamard import hadamard128_fp32_order


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


def expert_ffn(x_bits, topk_ids, topk_w, E, gate_fns, up_fns, down_fns, down_signs):
    """FP64 y [T, H] of the routed expert FFN.

    x_bits: bf16 patterns [T, H] of the (rotated) input. gate_fns, up_fns, down_fns:
    (weight_of, scale_of) pairs as for expert_gemm (gate/up [I, H], down [H, I]).
    down_signs: int8 [I] or None. topk_w: [T, topk] or None.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    g = expert_gemm(x_bits, ids, None, E, *gate_fns)            # [T, topk, I]
    u = expert_gemm(x_bits, ids, None, E, *up_fns)
    I = g.shape[2]
    h = silu(g) * u
    h_bits = f32_to_bf16_bits_rne(h.astype(np.float32)).reshape(T * topk, I)
    h_rot = hadamard128_fp32_order(h_bits, down_signs)
    gates = None if topk_w is None else np.asarray(topk_w, dtype=np.float64).reshape(T * topk, 1)
    z = expert_gemm(h_rot, ids.reshape(T * topk, 1), gates, E, *down_fns)  # [T*topk, 1, H]
    z = z.reshape(T, topk, -1)
    y = np.zeros((T, z.shape[2]), dtype=np.float64)
    for k in range(topk):
        y = y + z[:, k, :]
    return y
