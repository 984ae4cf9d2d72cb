"""Pins of the FP8 trellis operands (FORMAT F19): T16 values rounded to E4M3 and contracted
with MXFP8 activations.

- the rounding of every T16 value against torch's float8_e4m3fn cast (an independent
  implementation of the OCP format) and against values worked out by hand on the E4M3 grid;
- the error bound that 3 stored mantissa bits fix;
- closed forms: a unit whose streams are all zero bits (every q = -255) or all one bits
  (every q = 151) multiplies each token's MXFP8 activation sum by one constant;
- a scalar loop over a small layer (oracle.decode_unit_scalar and the scalar E4M3 decode).
"""

import numpy as np
import pytest

import oracle
from oracle import pool
from workloads import rng_for

torch = pytest.importorskip("torch")

Q = np.arange(-255, 256)


def test_every_t16_value_matches_torch_cast():
    got = oracle.t16_e4m3_codes(Q)
    ref = torch.from_numpy(Q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    vals = oracle.t16_e4m3(Q)
    assert np.array_equal(vals, torch.from_numpy(ref).view(torch.float8_e4m3fn).to(torch.float64).numpy())


# (q, E4M3 value) worked out on the grid: steps of 1 up to 16, 2 in [16, 32), 4 in [32, 64),
# 8 in [64, 128), 16 in [128, 256); a tie goes to the value whose 3 mantissa bits are even.
HAND = [(0, 0.0), (1, 1.0), (16, 16.0), (17, 16.0), (19, 20.0), (33, 32.0), (34, 32.0),
        (35, 36.0), (100, 96.0), (151, 144.0), (232, 224.0), (247, 240.0), (248, 256.0),
        (255, 256.0), (-255, -256.0), (-17, -16.0), (-151, -144.0)]


@pytest.mark.parametrize("q,v", HAND)
def test_hand_values(q, v):
    assert oracle.t16_e4m3(np.array([q]))[0] == v


def test_error_bound_and_exact_small_values():
    v = oracle.t16_e4m3(Q)
    assert np.array_equal(v[np.abs(Q) <= 16], Q[np.abs(Q) <= 16])
    assert np.all(np.abs(v - Q) <= np.abs(Q) * 2.0 ** -4)
    assert np.all(np.sign(v) == np.sign(Q))
    with pytest.raises(ValueError):
        oracle.t16_e4m3(np.array([256]))


def _const_layer(word, K=3, E=2, out=32, inp=256):
    n = out * inp * K // 32
    rng = rng_for(730, 0)
    return {"E": E, "out": out, "in": inp, "layout": 0,
            "bits": np.full(E, K, np.uint8),
            "code_off": (np.arange(E, dtype=np.int64) * n * 4),
            "codes": np.full(E * n, word, dtype=np.uint32),
            "scales": rng.integers(0x3800, 0x3C00, (E, out)).astype(np.uint16),
            "signs": None, "out_signs": None}


@pytest.mark.parametrize("word,qv", [(0x00000000, -256.0), (0xFFFFFFFF, 144.0)])
def test_constant_streams_closed_form(word, qv):
    lay = _const_layer(word)
    rng = rng_for(730, 1)
    T, topk = 6, 2
    x = oracle.f32_to_bf16_bits_rne(rng.standard_normal((T, lay["in"])).astype(np.float32))
    ids = rng.integers(0, lay["E"], (T, topk)).astype(np.int32)
    ids[0, 1] = -1
    y = pool.trellis_slots(lay, x, ids, workers=2, fp8=True)
    xs = oracle.mxfp8_values(oracle.bf16_bits_to_f64(x)).sum(axis=1)
    sc = oracle.f16_bits_to_f64(lay["scales"])
    for t in range(T):
        for k in range(topk):
            e = ids[t, k]
            want = np.zeros(lay["out"]) if e < 0 else sc[e] * qv * xs[t]
            assert np.allclose(y[t, k], want, rtol=1e-12, atol=0)


def test_scalar_loop_small_layer():
    rng = rng_for(730, 2)
    K, E, out, inp = 2, 2, 32, 256
    n = out * inp * K // 32
    lay = {"E": E, "out": out, "in": inp, "layout": 0, "bits": np.full(E, K, np.uint8),
           "code_off": np.arange(E, dtype=np.int64) * n * 4,
           "codes": rng.integers(0, 2 ** 32, E * n, dtype=np.uint64).astype(np.uint32),
           "scales": rng.integers(0x2000, 0x2400, (E, out)).astype(np.uint16),
           "signs": None, "out_signs": None}
    T, topk = 3, 2
    x = oracle.f32_to_bf16_bits_rne(rng.standard_normal((T, inp)).astype(np.float32))
    ids = np.array([[0, 1], [1, -1], [0, 0]], dtype=np.int32)
    y = pool.trellis_slots(lay, x, ids, workers=2, fp8=True)
    xq = oracle.mxfp8_values(oracle.bf16_bits_to_f64(x))
    sc = oracle.f16_bits_to_f64(lay["scales"])
    for e in range(E):
        q = oracle.decode_unit_scalar(lay["codes"][e * n:(e + 1) * n], K, out, inp)  # [out][in]
        w = [[oracle.e4m3_value(int(oracle.t16_e4m3_codes(np.array([q[o][i]]))[0]))
              for o in range(out)] for i in range(inp)]
        for t in range(T):
            for k in range(topk):
                if ids[t, k] != e:
                    continue
                for o in range(0, out, 7):
                    acc = 0.0
                    for i in range(inp):
                        acc += xq[t, i] * w[i][o]
                    assert abs(y[t, k, o] - sc[e, o] * acc) <= 1e-12 * max(1.0, abs(sc[e, o] * acc))
    assert np.all(y[1, 1] == 0)
