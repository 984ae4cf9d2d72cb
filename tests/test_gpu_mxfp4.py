"""MXFP4 expert GEMV / GEMM on the GPU vs the FP64 oracle (relative L2 <= 1e-3)."""

import numpy as np
import pytest

from gpu_helpers import gpu, needs_gpu, ops, oracle_mxfp4, rel_l2, slot_errors, to_dev, torch
from workloads import (bf16_from_normal, mxfp4_decode_layer, mxfp4_layer, mxfp4_prefill_chunk,
                       rng_for, softmax_gates, uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def run(layer_h, x_bits, ids, gates=None, flags=0):
    o = ops()
    L = o.Mxfp4Layer.from_host(layer_h)
    y = o.mxfp4_expert_gemm(L, to_dev(x_bits, np.int16), to_dev(ids),
                            None if gates is None else to_dev(gates), flags=flags)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("flags", [1, 2, 1 | 4, 2 | 4])
def test_small_layer(flags):
    E, T, topk = 7, 45, 3
    layer = mxfp4_layer(500, E, 256, 1024)
    x = bf16_from_normal(rng_for(500, 1), (T, 1024))
    ids = uniform_routes(rng_for(500, 2), T, E, topk)
    ids[4, 2] = -1
    gates = softmax_gates(rng_for(500, 3), T, topk)
    y = run(layer, x, ids, gates, flags=flags)
    ref = oracle_mxfp4(layer, x, ids, gates)
    if flags & 4:
        ref = ref.sum(axis=1)
    assert rel_l2(y, ref) <= TOL


def test_decode_layer_full_size():
    wl = mxfp4_decode_layer()
    y = run(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"])
    ref = oracle_mxfp4(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"])
    assert rel_l2(y, ref) <= TOL
    y2 = run(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"], flags=2)
    assert rel_l2(y2, ref) <= TOL


def test_long_pieces_sampled():
    # More expert groups (320 x 8) than the plan's wave target: each group is one piece of
    # 12 steps (or, on a GPU with a larger target, two of 6), so a piece spans several of the
    # kernel's 4-step scale blocks, starting at steps that are not multiples of 4.
    E, T, topk, out, inputs = 320, 256, 8, 1024, 1536
    layer = mxfp4_layer(501, E, out, inputs)
    x = bf16_from_normal(rng_for(501, 1), (T, inputs))
    ids = uniform_routes(rng_for(501, 2), T, E, topk)
    gates = softmax_gates(rng_for(501, 3), T, topk)
    y = run(layer, x, ids, gates)
    sample = np.sort(rng_for(501, 4).choice(T * topk, 48, replace=False))
    ref = oracle_mxfp4(layer, x, ids, gates, sample=sample)
    got = y.reshape(-1, out)[sample]
    assert rel_l2(got, ref.reshape(-1, out)[sample]) <= TOL


def test_deterministic():
    wl = mxfp4_decode_layer(E=64, T=32)
    a = run(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"])
    b = run(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"])
    assert np.array_equal(a, b)


def run_layer(L, x_bits, ids, gates=None, flags=0):
    o = ops()
    y = o.mxfp4_expert_gemm(L, to_dev(x_bits, np.int16), to_dev(ids),
                            None if gates is None else to_dev(gates), flags=flags)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("flags", [1, 2, 1 | 4, 2 | 4])
def test_repacked_layout_is_bit_equal(flags):
    # 208 output channels: one full group of 8 strips and a partial group of 5
    E, T, topk = 7, 45, 3
    layer = mxfp4_layer(502, E, 208, 1024)
    x = bf16_from_normal(rng_for(502, 1), (T, 1024))
    ids = uniform_routes(rng_for(502, 2), T, E, topk)
    gates = softmax_gates(rng_for(502, 3), T, topk)
    L = ops().Mxfp4Layer.from_host(layer)
    P = L.repacked()
    assert P.layout == ops().TQ_LAYOUT_GEMV
    a = run_layer(L, x, ids, gates, flags)
    b = run_layer(P, x, ids, gates, flags)
    assert np.array_equal(a, b)
    ref = oracle_mxfp4(layer, x, ids, gates)
    assert rel_l2(b, ref.sum(axis=1) if flags & 4 else ref) <= TOL


def test_repacked_full_size_decode():
    wl = mxfp4_decode_layer()
    L = ops().Mxfp4Layer.from_host(wl["layer"])
    a = run_layer(L, wl["x"], wl["topk_ids"], wl["topk_w"])
    b = run_layer(L.repacked(), wl["x"], wl["topk_ids"], wl["topk_w"])
    assert np.array_equal(a, b)


@pytest.mark.timeout(900)
def test_prefill_chunk_full_size_every_slot():
    """The MXFP4 prefill chunk (384 units of 128 x 5120, 8,192 tokens, top-8 Zipf(1.1),
    gates) on the bf16 matrix cores, units repacked: every one of the 65,536 slots against
    the FP64 oracle."""
    o = ops()
    wl = mxfp4_prefill_chunk()
    L = o.Mxfp4Layer.from_host(wl["layer"]).repacked()
    y = o.mxfp4_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                            to_dev(wl["topk_w"]), flags=o.TQ_GEMM).cpu().numpy()
    ref = oracle_mxfp4(wl["layer"], wl["x"], wl["topk_ids"], wl["topk_w"])
    pooled, worst = slot_errors(y, ref)
    print("MXFP4 bf16 prefill, 65536 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL
