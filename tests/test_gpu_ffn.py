"""Routed expert FFN on the GPU (trellis_expert_ffn) vs the FP64 oracle (FORMAT F15, F2b,
F17): relative L2 <= 1e-3 pooled and per token, in both modes, with gates, empty slots, the
input rotation, output-side rotations, the down projection in the page's 128-input units
or in one strip-major unit, and layers repacked into the kernels' read order."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import gpu, needs_gpu, ops, slot_errors, to_dev, torch, trellis_weight_fns
from workloads import (bf16_from_normal, ffn_decode, ffn_layers, rng_for, softmax_gates,
                       uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def run(gate_up, down, x, ids, gates, flags, repack=False):
    o = ops()
    GU, D = (o.TrellisLayer.from_host(l) for l in (gate_up, down))
    if repack:
        GU, D = GU.repacked(), D.repacked()
    y = o.trellis_expert_ffn(GU, D, to_dev(x, np.int16), to_dev(ids),
                             None if gates is None else to_dev(gates), flags=flags | o.TQ_ROTATE)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def reference(gate_up, down, x, ids, gates):
    x_rot = oracle.hadamard128_fp32_order(x, gate_up["signs"])
    return oracle.expert_ffn(x_rot, ids, gates, gate_up["E"], trellis_weight_fns(gate_up),
                             trellis_weight_fns(down), down["signs"], gate_up.get("out_signs"),
                             down.get("out_signs"))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("units128", [True, False])
@pytest.mark.parametrize("out_rotation", [False, True])
def test_small_ffn(mode, units128, out_rotation):
    E, H, I, T, topk = 6, 512, 256, 24, 3
    widths = np.array([2, 3, 4, 2, 2, 3], dtype=np.uint8)
    gate_up, down = ffn_layers(710, widths, H, I, down_units128=units128, out_rotation=out_rotation)
    x = bf16_from_normal(rng_for(710, 3), (T, H))
    ids = uniform_routes(rng_for(710, 4), T, E, topk)
    ids[5, 1] = -1
    gates = softmax_gates(rng_for(710, 5), T, topk)
    y = run(gate_up, down, x, ids, gates, mode)
    ref = reference(gate_up, down, x, ids, gates)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL, (pooled, worst)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("mode", [1, 2])
def test_ffn_repacked_layers_give_the_same_bits(mode):
    E, H, I, T, topk = 5, 512, 256, 16, 2
    widths = np.array([2, 3, 4, 2, 3], dtype=np.uint8)
    gate_up, down = ffn_layers(712, widths, H, I, out_rotation=True)
    x = bf16_from_normal(rng_for(712, 3), (T, H))
    ids = uniform_routes(rng_for(712, 4), T, E, topk)
    gates = softmax_gates(rng_for(712, 5), T, topk)
    a = run(gate_up, down, x, ids, gates, mode)
    b = run(gate_up, down, x, ids, gates, mode, repack=True)
    assert np.array_equal(a, b)


def test_ffn_bad_id_gives_nan_rows():
    E, H, I, T, topk = 4, 256, 256, 6, 2
    gate_up, down = ffn_layers(713, np.array([2, 2, 3, 4], np.uint8), H, I)
    x = bf16_from_normal(rng_for(713, 3), (T, H))
    ids = uniform_routes(rng_for(713, 4), T, E, topk)
    ids[2, 1] = 9
    for mode in (1, 2):
        y = run(gate_up, down, x, ids, None, mode)
        assert np.all(np.isnan(y[2]))
        keep = np.arange(T) != 2
        ref = reference(gate_up, down, x[keep], ids[keep], None)
        pooled, worst = slot_errors(y[keep], ref)
        assert worst <= TOL, (mode, worst)


def test_ffn_decode_shapes_sampled_experts():
    # the decode FFN's shapes (H = 5120, I = 768, 6 units of 128 intermediate channels per
    # projection), routes over 2 of 8 experts so that the FP64 oracle stays within seconds
    wl = ffn_decode(E=8, T=8, topk=2)
    ids = uniform_routes(rng_for(711, 0), 8, 2, 2)
    gates = wl["topk_w"]
    for mode in (1, 2):
        y = run(wl["gate_up"], wl["down"], wl["x"], ids, gates, mode)
        ref = reference(wl["gate_up"], wl["down"], wl["x"], ids, gates)
        pooled, worst = slot_errors(y, ref)
        assert pooled <= TOL and worst <= TOL, (mode, pooled, worst)


@pytest.mark.timeout(900)
def test_ffn_decode_full_workload():
    """The FFN decode workload at full size (384 experts, the fused gate/up 1536 x 5120 and
    the down 5120 x 768 in units of 128 intermediate channels, mixed widths, 128 tokens,
    top-8, gates, the input rotation fused): every output of every token against the FP64
    oracle."""
    wl = ffn_decode()
    y = run(wl["gate_up"], wl["down"], wl["x"], wl["topk_ids"], wl["topk_w"], 0, repack=True)
    x_rot = oracle.hadamard128_fp32_order(wl["x"], wl["gate_up"]["signs"])
    ref = oracle_pool.ffn(wl["gate_up"], wl["down"], x_rot, wl["topk_ids"], wl["topk_w"])
    pooled, worst = slot_errors(y, ref)
    print("FFN decode, 128 tokens x 5120: pooled %.3e, worst token %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL
