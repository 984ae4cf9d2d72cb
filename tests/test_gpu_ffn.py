"""Routed expert FFN on the GPU (trellis_expert_ffn) vs the FP64 oracle (FORMAT F15):
relative L2 <= 1e-3, in both modes, with gates, empty slots and the input rotation."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import gpu, needs_gpu, ops, rel_l2, slot_errors, to_dev, torch, trellis_weight_fns
from workloads import (bf16_from_normal, ffn_decode, ffn_layers, mixed_widths, rng_for,
                       softmax_gates, uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def run(gate, up, down, x, ids, gates, flags):
    o = ops()
    G, U, D = (o.TrellisLayer.from_host(l) for l in (gate, up, down))
    y = o.trellis_expert_ffn(G, U, D, to_dev(x, np.int16), to_dev(ids),
                             None if gates is None else to_dev(gates), flags=flags | o.TQ_ROTATE)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def reference(gate, up, down, x, ids, gates):
    x_rot = oracle.hadamard128_fp32_order(x, gate["signs"])
    return oracle.expert_ffn(x_rot, ids, gates, gate["E"], trellis_weight_fns(gate),
                             trellis_weight_fns(up), trellis_weight_fns(down), down["signs"])


@pytest.mark.parametrize("mode", [1, 2])
def test_small_ffn(mode):
    E, H, I, T, topk = 6, 512, 256, 24, 3
    widths = np.array([2, 3, 4, 2, 2, 3], dtype=np.uint8)
    gate, up, down = ffn_layers(710, widths, H, I)
    x = bf16_from_normal(rng_for(710, 3), (T, H))
    ids = uniform_routes(rng_for(710, 4), T, E, topk)
    ids[5, 1] = -1
    gates = softmax_gates(rng_for(710, 5), T, topk)
    y = run(gate, up, down, x, ids, gates, mode)
    ref = reference(gate, up, down, x, ids, gates)
    assert rel_l2(y, ref) <= TOL
    assert np.isfinite(y).all()


def test_ffn_decode_shapes_sampled_experts():
    # the decode FFN's shapes (H = 5120, I = 768, 6 units of 128 intermediate channels per
    # projection), routes over 2 of 8 experts so that the FP64 oracle stays within seconds
    wl = ffn_decode(E=8, T=8, topk=2)
    ids = uniform_routes(rng_for(711, 0), 8, 2, 2)
    gates = wl["topk_w"]
    y = run(wl["gate"], wl["up"], wl["down"], wl["x"], ids, gates, 0)
    ref = reference(wl["gate"], wl["up"], wl["down"], wl["x"], ids, gates)
    assert rel_l2(y, ref) <= TOL

