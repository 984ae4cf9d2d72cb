"""Pins of the FFN oracle (FORMAT F15): the gated activation against its closed forms and a
second, scalar implementation; the composition against a scalar brute force on a tiny FFN;
the combine's linearity in the gates and the empty slot."""

import math

import numpy as np
import pytest

import oracle
from workloads import bf16_from_normal, rng_for


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # sigma(ln 3) = 3/4
    assert oracle.silu(np.array([math.log(3.0)]))[0] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    # silu(a) - silu(-a) = a (sigma(a) + sigma(-a) = 1)
    a = rng_for(700, 0).standard_normal(1000) * 8.0
    assert np.allclose(oracle.silu(a) - oracle.silu(-a), a, rtol=1e-13, atol=1e-13)
    # far tails: silu(a) -> a for large a, -> 0 for very negative a
    assert oracle.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-20)
    assert abs(oracle.silu(np.array([-60.0]))[0]) < 1e-24


def test_silu_against_scalar_definition():
    a = rng_for(700, 1).standard_normal(2000) * 6.0
    got = oracle.silu(a)
    ref = np.array([oracle.silu_scalar(float(v)) for v in a])
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


def _tiny_ffn():
    """E = 2 experts, H = I = 128, integer weights in [-3, 3], scales 1/64 and 1/32."""
    rng = rng_for(701, 0)
    E, H, I = 2, 128, 128
    wg = rng.integers(-3, 4, size=(E, I, H)).astype(np.float64)
    wu = rng.integers(-3, 4, size=(E, I, H)).astype(np.float64)
    wd = rng.integers(-3, 4, size=(E, H, I)).astype(np.float64)
    sg = np.full((E, I), 1 / 64.0)
    sd = np.full((E, H), 1 / 32.0)
    signs = np.where(rng.integers(0, 2, size=I) == 1, 1, -1).astype(np.int8)
    fns = lambda w, s: (lambda e: w[e], lambda e: s[e])
    return E, H, I, fns(wg, sg), fns(wu, sg), fns(wd, sd), signs, (wg, wu, wd, sg, sd)


def test_composition_against_scalar_brute_force():
    E, H, I, gf, uf, df, signs, (wg, wu, wd, sg, sd) = _tiny_ffn()
    x = bf16_from_normal(rng_for(701, 1), (2, H))
    ids = np.array([[0, 1], [1, -1]], dtype=np.int32)
    gates = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    y = oracle.expert_ffn(x, ids, gates, E, gf, uf, df, signs)
    xv = oracle.bf16_bits_to_f64(x)
    for t in range(2):
        ref = [0.0] * H
        for k in range(2):
            e = int(ids[t, k])
            if e < 0:
                continue
            h = []
            for i in range(I):
                gv = sum(xv[t, j] * wg[e, i, j] for j in range(H)) * sg[e, i]
                uv = sum(xv[t, j] * wu[e, i, j] for j in range(H)) * sg[e, i]
                h.append(oracle.silu_scalar(gv) * uv)
            hb = oracle.f32_to_bf16_bits_rne(np.array(h, dtype=np.float32)).reshape(1, I)
            hr = oracle.bf16_bits_to_f64(oracle.hadamard128_fp32_order(hb, signs))[0]
            for o in range(H):
                z = sum(hr[i] * wd[e, o, i] for i in range(I)) * sd[e, o]
                ref[o] += float(gates[t, k]) * z
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-9), t


def test_linear_in_gates_and_empty_slots():
    E, H, I, gf, uf, df, signs, _ = _tiny_ffn()
    x = bf16_from_normal(rng_for(701, 2), (3, H))
    ids = np.array([[0, 1], [1, 0], [-1, -1]], dtype=np.int32)
    g1 = np.array([[0.5, 0.25], [1.0, 0.125], [1.0, 1.0]], dtype=np.float32)
    y1 = oracle.expert_ffn(x, ids, g1, E, gf, uf, df, signs)
    y2 = oracle.expert_ffn(x, ids, g1 * 2, E, gf, uf, df, signs)
    assert np.array_equal(y2, 2 * y1)  # doubling is exact in FP64
    assert np.all(y1[2] == 0.0)        # a token with only empty slots
    # one slot alone equals the two-slot sum minus the other slot
    ya = oracle.expert_ffn(x[:1], ids[:1, :1], g1[:1, :1], E, gf, uf, df, signs)
    yb = oracle.expert_ffn(x[:1], ids[:1, 1:], g1[:1, 1:], E, gf, uf, df, signs)
    assert np.allclose(y1[0], ya[0] + yb[0], rtol=1e-13, atol=1e-12)
