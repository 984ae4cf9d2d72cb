"""Prefill routing shapes that exercise how the route scan lays out the work items: items of
experts with many slots placed by token range, the other items filling equal XCD segments,
and the snake order within segments (one-group layers). Whatever the layout, every routed
slot must be computed once, by its own expert: every slot is compared with the FP64 oracle
(per-slot and pooled relative L2 <= 1e-3). The shapes: every token on the same two experts
(all items in one range), fewer rank blocks than token ranges (empty ranges), a block count
that is neither a multiple of 8 nor of the scan's batch, more blocks than one batch, more
items than one round of the snake ordering, 1,024 experts (the largest that is placed by
range) and 1,025 (the plain layout), several output groups (no snake order), and the MXFP4
prefill with gates."""

import numpy as np
import pytest

from gpu_helpers import (gpu, needs_gpu, ops, oracle_mxfp4, oracle_trellis, slot_errors, to_dev,
                         torch)
from workloads import (bf16_from_normal, mxfp4_layer, rng_for, softmax_gates, trellis_layer,
                       zipf_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def _trellis(seed, E, T, topk, ids, out=128, inp=256):
    o = ops()
    widths = rng_for(seed, 9).integers(2, 5, size=E).astype(np.uint8)
    layer = trellis_layer(seed, widths, out, inp, with_signs=True)
    x = bf16_from_normal(rng_for(seed, 1), (T, inp))
    L = o.TrellisLayer.from_host(layer)
    y = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), flags=o.TQ_GEMM)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref = oracle_trellis(layer, x, ids, None)
    assert not np.isnan(y).any()
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL, (pooled, worst)


def test_every_token_on_the_same_two_experts():
    T, E, topk = 700, 4, 2
    ids = np.tile(np.array([[1, 0]], dtype=np.int32), (T, 1))
    _trellis(1100, E, T, topk, ids)


def test_fewer_rank_blocks_than_ranges():
    T, E, topk = 1000, 64, 8  # 8,000 slots: 4 rank blocks of 2,048
    _trellis(1101, E, T, topk, zipf_routes(rng_for(1101, 2), T, E, topk))


def test_block_count_not_a_multiple_of_8_or_32():
    T, E, topk = 4100, 256, 8  # 32,800 slots: 17 rank blocks
    _trellis(1102, E, T, topk, zipf_routes(rng_for(1102, 2), T, E, topk))


def test_more_rank_blocks_than_one_scan_batch():
    T, E, topk = 10000, 128, 8  # 80,000 slots: 40 rank blocks, range starts in two batches
    _trellis(1106, E, T, topk, zipf_routes(rng_for(1106, 2), T, E, topk))


@pytest.mark.timeout(600)
def test_item_list_longer_than_one_ordering_round():
    T, E, topk = 20000, 64, 8  # 160,000 slots: over 1,024 items, two rounds of the ordering
    _trellis(1107, E, T, topk, zipf_routes(rng_for(1107, 2), T, E, topk))


@pytest.mark.parametrize("E", [1024, 1025])
def test_most_experts_placed_by_range_and_beyond(E):
    T, topk = 2048, 8
    _trellis(1103, E, T, topk, zipf_routes(rng_for(1103, 2), T, E, topk))


def test_several_output_groups():
    T, E, topk = 1500, 48, 4
    _trellis(1104, E, T, topk, zipf_routes(rng_for(1104, 2), T, E, topk), out=384)


def test_mxfp4_prefill_with_gates():
    o = ops()
    T, E, topk, out, inp = 3000, 96, 8, 128, 512
    layer = mxfp4_layer(1105, E, out, inp)
    x = bf16_from_normal(rng_for(1105, 1), (T, inp))
    ids = zipf_routes(rng_for(1105, 2), T, E, topk)
    gates = softmax_gates(rng_for(1105, 3), T, topk)
    y = o.mxfp4_expert_gemm(o.Mxfp4Layer.from_host(layer), to_dev(x, np.int16), to_dev(ids),
                            to_dev(gates), flags=o.TQ_GEMM)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref = oracle_mxfp4(layer, x, ids, gates)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL, (pooled, worst)
