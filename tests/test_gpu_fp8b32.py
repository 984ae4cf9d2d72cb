"""fp8b32 expert store on the GPU (FORMAT F16): the device decoder bit for bit against the
oracle, and the GEMV / GEMM through fp8b32_expert_gemm against the FP64 oracle
(relative L2 <= 1e-3)."""

import numpy as np
import pytest

import oracle
from gpu_helpers import gpu, needs_gpu, ops, rel_l2, to_dev, torch
from workloads import bf16_from_normal, fp8b32_layer, rng_for, shared_expert, softmax_gates, uniform_routes

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def decode(unit, out, inp):
    return ops().fp8b32_decode(to_dev(unit), out, inp).cpu().numpy().view(np.uint16)


def test_decode_unit():
    lay = fp8b32_layer(910, 1, 128, 5120)
    w = decode(lay["units"], 128, 5120)
    ref = oracle.f64_to_bf16_bits_exact(oracle.decode_fp8b32_unit(lay["units"], 128, 5120))
    assert np.array_equal(w, ref)


def test_decode_every_code_over_the_exact_scale_range():
    # 8 row blocks x 256 column blocks; block (rb, cb) takes scale byte 10 + (256 rb + cb) % 237
    # (10 .. 246, where every product is a normal bf16); row r holds codes (i + 7 r) % 256,
    # so every code, the two NaN codes among them, meets many scales
    out, inp = 256, 8192
    i = np.arange(inp)[None, :]
    r = np.arange(out)[:, None]
    codes = ((i + 7 * r) % 256).astype(np.uint8)
    blk = np.arange(8)[:, None] * 256 + np.arange(256)[None, :]
    scales = (10 + blk % 237).astype(np.uint8)
    unit = np.concatenate([codes.reshape(-1), scales.reshape(-1)])
    w = decode(unit, out, inp)
    vals = oracle.decode_fp8b32_unit(unit, out, inp)
    nan = np.isnan(vals)
    assert nan.any() and np.array_equal(np.isnan(oracle.bf16_bits_to_f64(w)), nan)
    ref = oracle.f64_to_bf16_bits_exact(np.where(nan, 0.0, vals))
    mismatch = np.argwhere((w != ref) & ~nan)
    assert mismatch.size == 0, mismatch[:8]


def test_decode_nan_scale():
    out, inp = 32, 64
    unit = np.full(out * inp + 2, 0x38, dtype=np.uint8)   # every code 1.0
    unit[-2:] = (127, 255)                                # block 1 has the NaN scale
    w = oracle.bf16_bits_to_f64(decode(unit, out, inp))
    assert (w[:, :32] == 1.0).all() and np.isnan(w[:, 32:]).all()


def fp8b32_weight_fn(layer):
    ub = oracle.fp8b32_unit_bytes(layer["out"], layer["in"])
    units = layer["units"].reshape(layer["E"], ub)
    cache = {}

    def weight_of(e):
        if e not in cache:
            cache[e] = oracle.decode_fp8b32_unit(units[e], layer["out"], layer["in"])
        return cache[e]
    return weight_of


def run(layer_h, x_bits, ids, gates=None, flags=0):
    o = ops()
    L = o.Fp8b32Layer.from_host(layer_h)
    y = o.fp8b32_expert_gemm(L, to_dev(x_bits, np.int16), to_dev(ids),
                             None if gates is None else to_dev(gates), flags=flags)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def reference(layer, x_bits, ids, gates):
    return oracle.expert_gemm(x_bits, np.asarray(ids), gates, layer["E"], fp8b32_weight_fn(layer), None)


@pytest.mark.parametrize("flags", [1, 2, 1 | 4, 2 | 4])
def test_small_layer(flags):
    # 7 experts of 96 x 1024 (3 row blocks, a ragged last strip group), 45 tokens, top-3,
    # one empty slot, gates
    E, T, topk = 7, 45, 3
    layer = fp8b32_layer(911, E, 96, 1024)
    x = bf16_from_normal(rng_for(911, 1), (T, 1024))
    ids = uniform_routes(rng_for(911, 2), T, E, topk)
    ids[4, 2] = -1
    gates = softmax_gates(rng_for(911, 3), T, topk)
    y = run(layer, x, ids, gates, flags=flags)
    ref = reference(layer, x, ids, gates)
    if flags & 4:
        ref = ref.sum(axis=1)
    assert rel_l2(y, ref) <= TOL


@pytest.mark.parametrize("T, flags", [(128, 0), (128, 2), (1024, 0), (1024, 2), (4096, 0)])
def test_shared_expert(T, flags):
    # the shared expert's gate and up projections (1536 x 5120), every token routed to it:
    # up to 2048 tokens take the decode batch by default (their 12 x T/128 prefill items are
    # fewer than the GPU's compute units), 4096 the prefill GEMM; flags 2 forces the GEMM
    wl = shared_expert(T=T)
    y = run(wl["layer"], wl["x"], wl["topk_ids"], None, flags=flags)
    ref = reference(wl["layer"], wl["x"], wl["topk_ids"], None)
    assert rel_l2(y, ref) <= TOL
    # every output row is the x row times the decoded matrix, whichever mode ran
    assert y.shape == (T, 1, 1536)


def test_deterministic():
    wl = shared_expert(T=64)
    a = run(wl["layer"], wl["x"], wl["topk_ids"])
    b = run(wl["layer"], wl["x"], wl["topk_ids"])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("flags", [1, 2, 1 | 4])
def test_repacked_layout_is_bit_equal(flags):
    # 224 output channels: one full group of 8 strips and a partial group of 6
    E, T, topk = 5, 40, 2
    layer = fp8b32_layer(912, E, 224, 1024)
    x = bf16_from_normal(rng_for(912, 1), (T, 1024))
    ids = uniform_routes(rng_for(912, 2), T, E, topk)
    gates = softmax_gates(rng_for(912, 3), T, topk)
    o = ops()
    L = o.Fp8b32Layer.from_host(layer)
    P = L.repacked()
    outs = []
    for lay in (L, P):
        y = o.fp8b32_expert_gemm(lay, to_dev(x, np.int16), to_dev(ids), to_dev(gates), flags=flags)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    ref = reference(layer, x, ids, gates)
    assert rel_l2(outs[1], ref.sum(axis=1) if flags & 4 else ref) <= TOL
