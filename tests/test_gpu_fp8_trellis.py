"""The FP8 trellis prefill (FORMAT F19) on the GPU against the oracle that emulates its two
roundings: the E4M3 operands of the weight decoder bit for bit (decode hook, path 2), and
the GEMM (relative L2 <= 1e-3 per slot and pooled against the FP64 contraction of the MXFP8
activations with the E4M3-rounded T16 values), in every code layout, with the rotation
fused, with combine, with empty, invalid and non-finite slots, and at full size."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import gpu, needs_gpu, ops, slot_errors, to_dev, torch
from workloads import (bf16_from_normal, prefill_chunk, random_words, rng_for, softmax_gates,
                       trellis_layer, uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


@pytest.mark.parametrize("K", [2, 3, 4])
def test_e4m3_decode_hook_unit(K):
    out, inp = 128, 5120
    words = random_words(rng_for(850, K), out * inp * K // 32)
    codes = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, 2).cpu().numpy()
    ref = oracle.t16_e4m3_codes(oracle.decode_unit(words, K, out, inp))
    assert np.array_equal(codes.astype(np.uint8), ref)
    assert np.all((codes >= 0) & (codes < 256))


@pytest.mark.parametrize("K", [2, 3, 4])
def test_e4m3_decode_hook_special_streams(K):
    out, inp = 32, 128
    n = out * inp * K // 32
    tile = np.array([(0x9E3779B9 * (j + 1)) % (1 << 32) for j in range(8 * K)], dtype=np.uint32)
    for words in (np.zeros(n, np.uint32), np.full(n, 0xFFFFFFFF, np.uint32),
                  np.tile(tile, n // tile.size)):
        codes = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, 2).cpu().numpy()
        ref = oracle.t16_e4m3_codes(oracle.decode_unit(words, K, out, inp))
        assert np.array_equal(codes.astype(np.uint8), ref)


def _layer(seed, E, out, inp, layout=0):
    widths = np.array([2, 3, 4] * ((E + 2) // 3), dtype=np.uint8)[:E]
    lay = trellis_layer(seed, widths, out, inp, with_signs=True)
    lay["layout"] = layout
    return lay


def _oracle(layer, x_bits, ids, gates, rotate):
    x = oracle.hadamard128_fp32_order(x_bits, layer["signs"]) if rotate else x_bits
    return oracle_pool.trellis_slots(layer, x, ids, gates, fp8=True)


@pytest.mark.parametrize("layout", ["store", "repacked", "unit128"])
@pytest.mark.parametrize("combine", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_trellis_fp8_prefill_small(layout, combine, rotate):
    o = ops()
    E, T, topk, inp, out = 9, 70, 4, 1024, 256
    layer = _layer(851, E, out, inp, o.TQ_LAYOUT_UNIT128 if layout == "unit128" else 0)
    x = bf16_from_normal(rng_for(851, 1), (T, inp))
    ids = uniform_routes(rng_for(851, 2), T, E, topk)
    ids[3, 1] = -1
    ids[7, 0] = 99  # invalid: NaN slot
    gates = softmax_gates(rng_for(851, 3), T, topk)
    L = o.TrellisLayer.from_host(layer)
    if layout == "repacked":
        L = L.repacked()
    flags = o.TQ_FP8 | (o.TQ_COMBINE if combine else 0) | (o.TQ_ROTATE if rotate else 0)
    y = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), to_dev(gates), flags=flags)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref = _oracle(layer, x, ids, gates, rotate)
    if combine:
        ref = oracle.combine_slots(ref)
        bad = np.zeros(T, bool)
        bad[7] = True
        assert np.all(np.isnan(y[bad]))
        y, ref = y[~bad], ref[~bad]
    else:
        assert np.all(np.isnan(y[7, 0])) and np.all(y[3, 1] == 0)
        keep = np.ones((T, topk), bool)
        keep[7, 0] = False
        y, ref = y[keep], ref[keep]
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL, (pooled, worst)


def test_trellis_fp8_non_finite_token_and_batch_invariance():
    """A token with an infinity gets NaN slots; every other slot has the same bits whether
    it runs in the whole batch or in a batch of its token alone."""
    o = ops()
    E, T, topk, inp = 6, 48, 3, 512
    layer = _layer(852, E, 128, inp)
    x = bf16_from_normal(rng_for(852, 1), (T, inp)).copy()
    x[9, 300] = 0x7F80
    ids = uniform_routes(rng_for(852, 2), T, E, topk)
    L = o.TrellisLayer.from_host(layer)
    y = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), flags=o.TQ_FP8).cpu().numpy()
    assert np.all(np.isnan(y[9]))
    keep = np.arange(T) != 9
    pooled, worst = slot_errors(y[keep], _oracle(layer, x[keep], ids[keep], None, False))
    assert pooled <= TOL and worst <= TOL
    for t in (0, 17, 47):
        y1 = o.trellis_expert_gemm(L, to_dev(x[t:t + 1], np.int16), to_dev(ids[t:t + 1]),
                                   flags=o.TQ_FP8).cpu().numpy()
        assert np.array_equal(y1[0], y[t])


def test_trellis_fp8_rejects_decode_mode():
    o = ops()
    layer = _layer(853, 3, 128, 512)
    x = to_dev(bf16_from_normal(rng_for(853, 1), (4, 512)), np.int16)
    ids = to_dev(uniform_routes(rng_for(853, 2), 4, 3, 2))
    with pytest.raises(RuntimeError):
        o.trellis_expert_gemm(o.TrellisLayer.from_host(layer), x, ids, flags=o.TQ_FP8 | o.TQ_GEMV)


@pytest.mark.timeout(900)
def test_trellis_fp8_prefill_full_size_every_slot():
    """The prefill chunk (8,192 tokens, top-8, 384 K=3 experts, Zipf(1.1), the rotation
    fused) on the fp8 matrix cores, units repacked: every one of the 65,536 slots against
    the oracle's MXFP8 x E4M3 contraction."""
    o = ops()
    wl = prefill_chunk()
    layer = wl["layer"]
    L = o.TrellisLayer.from_host(layer).repacked()
    y = o.trellis_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                              flags=o.TQ_FP8 | o.TQ_ROTATE).cpu().numpy()
    ref = _oracle(layer, wl["x"], wl["topk_ids"], None, True)
    pooled, worst = slot_errors(y, ref)
    print("trellis FP8 prefill, 65536 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL
