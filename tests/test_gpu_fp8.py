"""FP8 matrix-core variants (FORMAT F18) on the GPU against the oracle that emulates their
operand roundings: the MXFP8 activation conversion bit for bit, and the MXFP4 prefill on the
block-scaled fp8 x fp4 matrix cores (relative L2 <= 1e-3 against the FP64 contraction of the
MXFP8 activations with the exact MXFP4 weights)."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import gpu, needs_gpu, ops, slot_errors, to_dev, torch
from workloads import (bf16_from_normal, mxfp4_layer, mxfp4_prefill_chunk, rng_for,
                       softmax_gates, uniform_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def _bf16(v):
    f = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def test_mxfp8_quantize_bit_exact():
    rng = rng_for(800, 0)
    rows, n = 40, 2048
    xf = rng.standard_normal((rows, n)) * np.exp2(rng.integers(-60, 60, (rows, 1)))
    xf[1, 64:96] = 0.0                                 # an all-zero block
    xf[2, :] = rng.standard_normal(n) * 1e-38          # bf16 subnormals
    xf[3, 32:64] = np.where(np.arange(32) % 2, 3e38, -1e-3)
    x = _bf16(xf)
    x[4, 100] = 0x7F80                                 # +inf: NaN block
    x[5, 7] = 0x7FC0                                   # NaN
    codes, scales = ops().mxfp8_quantize(to_dev(x, np.int16))
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    ref_c, ref_s = oracle.quantize_mxfp8_rows(oracle.bf16_bits_to_f64(x))
    assert np.array_equal(scales, ref_s)
    finite_block = np.repeat(ref_s != 255, 32, axis=1)
    assert np.array_equal(codes[finite_block], ref_c[finite_block])


def _oracle_fp8(layer, x_bits, ids, gates):
    c, s = oracle.quantize_mxfp8_rows(oracle.bf16_bits_to_f64(x_bits))
    xq = oracle.dequantize_mxfp8_rows(c, s)
    return oracle_pool.mxfp4_slots(layer, xq, ids, gates)


@pytest.mark.parametrize("repack", [False, True])
@pytest.mark.parametrize("combine", [False, True])
def test_mxfp4_fp8_prefill_small(repack, combine):
    o = ops()
    E, T, topk, inp, out = 7, 90, 4, 1024, 384
    layer = mxfp4_layer(801, E, out, inp)
    x = bf16_from_normal(rng_for(801, 1), (T, inp))
    ids = uniform_routes(rng_for(801, 2), T, E, topk)
    ids[3, 1] = -1
    ids[7, 0] = 99  # invalid: NaN slot
    gates = softmax_gates(rng_for(801, 3), T, topk)
    L = o.Mxfp4Layer.from_host(layer)
    if repack:
        L = L.repacked()
    flags = o.TQ_FP8 | (o.TQ_COMBINE if combine else 0)
    y = o.mxfp4_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), to_dev(gates), flags=flags)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref = _oracle_fp8(layer, x, ids, gates)
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


def test_mxfp4_fp8_prefill_non_finite_token():
    o = ops()
    E, T, topk, inp = 5, 40, 2, 512
    layer = mxfp4_layer(802, E, 128, inp)
    x = bf16_from_normal(rng_for(802, 1), (T, inp)).copy()
    x[9, 300] = 0x7F80  # +inf: that token's slots are NaN
    ids = uniform_routes(rng_for(802, 2), T, E, topk)
    y = o.mxfp4_expert_gemm(o.Mxfp4Layer.from_host(layer), to_dev(x, np.int16), to_dev(ids),
                            flags=o.TQ_FP8).cpu().numpy()
    assert np.all(np.isnan(y[9]))
    keep = np.arange(T) != 9
    ref = _oracle_fp8(layer, x[keep], ids[keep], None)
    pooled, worst = slot_errors(y[keep], ref)
    assert pooled <= TOL and worst <= TOL


@pytest.mark.timeout(900)
def test_mxfp4_fp8_prefill_full_size_every_slot():
    """The MXFP4 prefill chunk (384 units of 128 x 5120, 8,192 tokens, top-8 Zipf(1.1),
    gates) on the fp8 matrix cores, units repacked: every one of the 65,536 slots against
    the oracle with the MXFP8 activations."""
    o = ops()
    wl = mxfp4_prefill_chunk()
    layer = wl["layer"]
    L = o.Mxfp4Layer.from_host(layer).repacked()
    y = o.mxfp4_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                            to_dev(wl["topk_w"]), flags=o.TQ_FP8)
    y = y.cpu().numpy()
    ref = _oracle_fp8(layer, wl["x"], wl["topk_ids"], wl["topk_w"])
    pooled, worst = slot_errors(y, ref)
    print("MXFP4 x MXFP8 prefill, 65536 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL
