"""The exlr8 codebooks on the GPU (FORMAT F20 mul1, F21 pmcgx): their FP8 operand decoders
bit for bit against the oracle (decode hook paths 3 and 4), and the FP8 prefill with each
codebook slot by slot against the oracle's MXFP8 x E4M3 contraction (relative L2 <= 1e-3),
including the prefill chunk at full size with a mul1 layer (the page's codebook of the K3
layers 8-37). Parity with real exlr8 files is unpinned (the readings of F20/F21)."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import gpu, needs_gpu, ops, slot_errors, to_dev, torch
from workloads import (bf16_from_normal, prefill_chunk, random_words, rng_for, softmax_gates,
                       trellis_layer, uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def _ref_codes(words, K, out, inp, codebook):
    if codebook == 1:
        return oracle.e4m3_round(oracle.decode_unit_mul1(words, K, out, inp) / 2.0)
    return oracle.decode_unit_pmcgx(words, K, out, inp)


@pytest.mark.parametrize("codebook", [1, 2])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_codebook_decode_hook_unit(codebook, K):
    out, inp = 128, 5120
    words = random_words(rng_for(860, codebook, K), out * inp * K // 32)
    codes = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, 2 + codebook).cpu().numpy()
    assert np.array_equal(codes.astype(np.uint8), _ref_codes(words, K, out, inp, codebook))


@pytest.mark.parametrize("codebook", [1, 2])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_codebook_decode_hook_special_streams(codebook, K):
    out, inp = 32, 128
    n = out * inp * K // 32
    tile = np.array([(0x9E3779B9 * (j + 1)) % (1 << 32) for j in range(8 * K)], dtype=np.uint32)
    for words in (np.zeros(n, np.uint32), np.full(n, 0xFFFFFFFF, np.uint32),
                  np.tile(tile, n // tile.size)):
        codes = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, 2 + codebook).cpu().numpy()
        assert np.array_equal(codes.astype(np.uint8), _ref_codes(words, K, out, inp, codebook))


def _layer(seed, codebook, E, out, inp):
    widths = np.array([2, 3, 4] * ((E + 2) // 3), dtype=np.uint8)[:E]
    lay = trellis_layer(seed, widths, out, inp, with_signs=True)
    lay["codebook"] = codebook
    return lay


@pytest.mark.parametrize("codebook", [1, 2])
@pytest.mark.parametrize("repack", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_codebook_fp8_prefill_small(codebook, repack, rotate):
    o = ops()
    E, T, topk, inp, out = 8, 60, 4, 768, 256
    layer = _layer(861, codebook, E, out, inp)
    x = bf16_from_normal(rng_for(861, 1), (T, inp))
    ids = uniform_routes(rng_for(861, 2), T, E, topk)
    ids[2, 3] = -1
    ids[5, 0] = 77
    gates = softmax_gates(rng_for(861, 3), T, topk)
    L = o.TrellisLayer.from_host(layer)
    if repack:
        L = L.repacked()
    flags = o.TQ_FP8 | (o.TQ_ROTATE if rotate else 0)
    y = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), to_dev(gates), flags=flags)
    y = y.cpu().numpy().astype(np.float64)
    xr = oracle.hadamard128_fp32_order(x, layer["signs"]) if rotate else x
    ref = oracle_pool.trellis_slots(layer, xr, ids, gates, fp8=True)
    assert np.all(np.isnan(y[5, 0])) and np.all(y[2, 3] == 0)
    keep = np.ones((T, topk), bool)
    keep[5, 0] = False
    pooled, worst = slot_errors(y[keep], ref[keep])
    assert pooled <= TOL and worst <= TOL, (pooled, worst)


def test_codebook_layers_need_fp8():
    o = ops()
    layer = _layer(862, 2, 3, 128, 512)
    x = to_dev(bf16_from_normal(rng_for(862, 1), (4, 512)), np.int16)
    ids = to_dev(uniform_routes(rng_for(862, 2), 4, 3, 2))
    with pytest.raises(RuntimeError):
        o.trellis_expert_gemm(o.TrellisLayer.from_host(layer), x, ids, flags=o.TQ_GEMM)


@pytest.mark.timeout(900)
def test_mul1_fp8_prefill_full_size_every_slot():
    """The prefill chunk (8,192 tokens, top-8, 384 K=3 experts, Zipf(1.1), rotation fused)
    stored with the mul1 codebook, units repacked: all 65,536 slots against the oracle."""
    o = ops()
    wl = prefill_chunk()
    layer = dict(wl["layer"], codebook=1)
    L = o.TrellisLayer.from_host(layer).repacked()
    y = o.trellis_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                              flags=o.TQ_FP8 | o.TQ_ROTATE).cpu().numpy()
    xr = oracle.hadamard128_fp32_order(wl["x"], layer["signs"])
    ref = oracle_pool.trellis_slots(layer, xr, wl["topk_ids"], None, fp8=True)
    pooled, worst = slot_errors(y, ref)
    print("mul1 FP8 prefill, 65536 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL
