"""The oracle's process pool (oracle/pool.py) against the same oracle calls made in one
process: splitting the routes by expert must not change a slot (the pool only decides where
each expert's slots are computed)."""

import numpy as np

import oracle
from oracle import pool
from workloads import (bf16_from_normal, ffn_layers, rng_for, softmax_gates, trellis_layer,
                       uniform_routes)


def _fns(layer):
    def weight_of(e):
        K = int(layer["bits"][e])
        n = layer["out"] * layer["in"] * K // 32
        s = int(layer["code_off"][e]) // 4
        return oracle.decode_unit(layer["codes"][s:s + n], K, layer["out"], layer["in"]).astype(np.float64)

    sc = oracle.f16_bits_to_f64(layer["scales"])
    return weight_of, lambda e: sc[e]


def test_pool_slots_equal_one_process():
    layer = trellis_layer(930, np.array([2, 3, 4, 2, 3, 2, 4], np.uint8), 32, 256, with_signs=False)
    x = bf16_from_normal(rng_for(930, 1), (12, 256))
    ids = uniform_routes(rng_for(930, 2), 12, 7, 3)
    ids[4, 2] = -1
    ids[5, 0] = 9  # invalid: NaN
    gates = softmax_gates(rng_for(930, 3), 12, 3)
    got = pool.trellis_slots(layer, x, ids, gates, workers=3)
    ref = oracle.expert_gemm(x, ids, gates, 7, *_fns(layer))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.allclose(np.nan_to_num(got), np.nan_to_num(ref), rtol=1e-13, atol=0)


def test_pool_ffn_equals_one_process():
    widths = np.array([2, 3, 4, 2], np.uint8)
    gate_up, down = ffn_layers(931, widths, 256, 256, down_units128=False, out_rotation=True)
    x = bf16_from_normal(rng_for(931, 1), (6, 256))
    ids = uniform_routes(rng_for(931, 2), 6, 4, 2)
    gates = softmax_gates(rng_for(931, 3), 6, 2)
    got = pool.ffn(gate_up, down, x, ids, gates, workers=2)
    ref = oracle.expert_ffn(x, ids, gates, 4, _fns(gate_up), _fns(down), down["signs"],
                            gate_up["out_signs"], down["out_signs"])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
