"""Pins of the FFN oracle (FORMAT F15, F2b, F17): the gated activation against its closed
forms and a second, scalar implementation; the rotations of FP64 values against explicit
matrix products and each other; the 128-input unit decode against tiles moved by hand; the
composition against a scalar brute force on a tiny FFN; the combine's linearity in the
gates and the empty slot."""

import math

import numpy as np
import pytest

import oracle
from workloads import bf16_from_normal, random_words, rng_for


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


def _explicit_rotation(signs):
    """The 128 x 128 matrix (1/sqrt(128)) H diag(s), H built entry by entry:
    H[i][j] = (-1)^popcount(i & j) (Sylvester, natural order)."""
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(128)] for i in range(128)],
                 dtype=np.float64)
    return H / math.sqrt(128.0) @ np.diag(np.asarray(signs, dtype=np.float64))


def test_rotations_of_values_against_explicit_matrices():
    rng = rng_for(702, 0)
    s = np.where(rng.integers(0, 2, 256) == 1, 1, -1).astype(np.int8)
    v = rng.standard_normal((3, 256))
    got_in = oracle.rotate128_values(v, s)
    got_out = oracle.output_rotation128(v, s)
    for b in range(2):
        R = _explicit_rotation(s[128 * b:128 * (b + 1)])
        blk = v[:, 128 * b:128 * (b + 1)]
        assert np.allclose(got_in[:, 128 * b:128 * (b + 1)], blk @ R.T, rtol=0, atol=1e-12)
        assert np.allclose(got_out[:, 128 * b:128 * (b + 1)], blk @ R, rtol=0, atol=1e-12)
    # the output rotation undoes the input rotation with the same signs (F17)
    assert np.allclose(oracle.output_rotation128(got_in, s), v, rtol=0, atol=1e-12)
    # on bf16 inputs the value rotation is the exact F8 transform
    xb = bf16_from_normal(rng_for(702, 1), (2, 256))
    assert np.array_equal(oracle.rotate128_values(oracle.bf16_bits_to_f64(xb), s),
                          oracle.hadamard128_f64(xb, s))


@pytest.mark.parametrize("K", [2, 3])
def test_units128_decode_against_moved_tiles(K):
    """A projection in 128-input units (F2b) holds the same tiles as the strip-major unit
    (F2): tile (to, ti) of the projection is tile (to, ti mod 8) of unit ti // 8. Moving the
    tile words by hand from one order to the other gives the same decoded matrix."""
    out, inp = 32, 384
    tw = 8 * K
    n_to, n_ti = out // 16, inp // 16
    words = random_words(rng_for(703, K), out * inp * K // 32)
    strip = words.reshape(n_to, n_ti, tw)
    units = np.empty((inp // 128, n_to, 8, tw), dtype=np.uint32)
    for to in range(n_to):
        for ti in range(n_ti):
            units[ti // 8, to, ti % 8] = strip[to, ti]
    q_units = oracle.decode_units128(units.reshape(-1), K, out, inp)
    assert np.array_equal(q_units, oracle.decode_unit(words, K, out, inp))
    # and unit j alone decodes to the inputs 128 j .. 128 j + 127
    per = out * 128 * K // 32
    for j in range(inp // 128):
        assert np.array_equal(oracle.decode_unit(units.reshape(-1)[j * per:(j + 1) * per], K, out, 128),
                              q_units[:, 128 * j:128 * (j + 1)])


def _tiny_ffn():
    """E = 2 experts, H = I = 128, integer weights in [-3, 3], scales 1/64 and 1/32; gate and
    up as one 2I x H projection (the gate's channels first)."""
    rng = rng_for(701, 0)
    E, H, I = 2, 128, 128
    wg = rng.integers(-3, 4, size=(E, I, H)).astype(np.float64)
    wu = rng.integers(-3, 4, size=(E, I, H)).astype(np.float64)
    wd = rng.integers(-3, 4, size=(E, H, I)).astype(np.float64)
    sgu = np.full((E, 2 * I), 1 / 64.0)
    sd = np.full((E, H), 1 / 32.0)
    signs = np.where(rng.integers(0, 2, size=I) == 1, 1, -1).astype(np.int8)
    wgu = np.concatenate([wg, wu], axis=1)
    fns = lambda w, s: (lambda e: w[e], lambda e: s[e])
    return E, H, I, fns(wgu, sgu), fns(wd, sd), signs, (wg, wu, wd)


def _brute(x_bits, ids, gates, wg, wu, wd, signs, sg, sd, gu_out=None, d_out=None):
    """The composition written out entry by entry (scalar Python, FP64)."""
    xv = oracle.bf16_bits_to_f64(x_bits)
    T, topk = ids.shape
    H, I = wd.shape[1], wd.shape[2]
    R = _explicit_rotation(signs)
    ys = []
    for t in range(T):
        ref = [0.0] * H
        for k in range(topk):
            e = int(ids[t, k])
            if e < 0:
                continue
            gv = [sum(xv[t, j] * wg[e, i, j] for j in range(H)) * sg for i in range(I)]
            uv = [sum(xv[t, j] * wu[e, i, j] for j in range(H)) * sg for i in range(I)]
            if gu_out is not None:  # F17 on the 2I outputs: blocks 0 (gate) and 1 (up)
                gv = list(np.array(gv) @ _explicit_rotation(gu_out[:I]))
                uv = list(np.array(uv) @ _explicit_rotation(gu_out[I:]))
            h = [oracle.silu_scalar(gv[i]) * uv[i] for i in range(I)]
            v = [sum(R[i, j] * h[j] for j in range(I)) for i in range(I)]
            z = [sum(v[i] * wd[e, o, i] for i in range(I)) * sd for o in range(H)]
            if d_out is not None:
                z = list(np.array(z) @ _explicit_rotation(d_out))
            for o in range(H):
                ref[o] += float(gates[t, k]) * z[o]
        ys.append(ref)
    return np.array(ys)


def test_composition_against_scalar_brute_force():
    E, H, I, guf, df, signs, (wg, wu, wd) = _tiny_ffn()
    x = bf16_from_normal(rng_for(701, 1), (2, H))
    ids = np.array([[0, 1], [1, -1]], dtype=np.int32)
    gates = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    y = oracle.expert_ffn(x, ids, gates, E, guf, df, signs)
    ref = _brute(x, ids, gates, wg, wu, wd, signs, 1 / 64.0, 1 / 32.0)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9)


def test_composition_with_output_rotations_against_brute_force():
    E, H, I, guf, df, signs, (wg, wu, wd) = _tiny_ffn()
    rng = rng_for(701, 5)
    gu_out = np.where(rng.integers(0, 2, size=2 * I) == 1, 1, -1).astype(np.int8)
    d_out = np.where(rng.integers(0, 2, size=H) == 1, 1, -1).astype(np.int8)
    x = bf16_from_normal(rng_for(701, 6), (1, H))
    ids = np.array([[1, 0]], dtype=np.int32)
    gates = np.array([[0.375, 0.625]], dtype=np.float32)
    y = oracle.expert_ffn(x, ids, gates, E, guf, df, signs, gu_out, d_out)
    ref = _brute(x, ids, gates, wg, wu, wd, signs, 1 / 64.0, 1 / 32.0, gu_out, d_out)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9)


def test_linear_in_gates_and_empty_slots():
    E, H, I, guf, df, signs, _ = _tiny_ffn()
    x = bf16_from_normal(rng_for(701, 2), (3, H))
    ids = np.array([[0, 1], [1, 0], [-1, -1]], dtype=np.int32)
    g1 = np.array([[0.5, 0.25], [1.0, 0.125], [1.0, 1.0]], dtype=np.float32)
    y1 = oracle.expert_ffn(x, ids, g1, E, guf, df, signs)
    y2 = oracle.expert_ffn(x, ids, g1 * 2, E, guf, df, signs)
    assert np.array_equal(y2, 2 * y1)  # doubling is exact in FP64
    assert np.all(y1[2] == 0.0)        # a token with only empty slots
    # one slot alone equals the two-slot sum minus the other slot
    ya = oracle.expert_ffn(x[:1], ids[:1, :1], g1[:1, :1], E, guf, df, signs)
    yb = oracle.expert_ffn(x[:1], ids[:1, 1:], g1[:1, 1:], E, guf, df, signs)
    assert np.allclose(y1[0], ya[0] + yb[0], rtol=1e-13, atol=1e-12)
