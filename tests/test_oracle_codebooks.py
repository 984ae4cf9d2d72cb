"""Pins of the exlr8 codebooks (FORMAT F20 mul1, F21 pmcgx). The page fixes the multipliers,
one weight per state for mul1, two weights per 20-bit state for pmcgx and the final E4M3
rounding; the rest are readings, so parity with real exlr8 files is unpinned. Pinned here:
- single states worked out by hand (tests/golden/exlr8_codebooks.txt);
- the pure-Python decoders (explicit bit lists) against the vectorised ones;
- the window structure: a single set bit of the stream changes exactly the states whose
  window covers it (16 bits at K p for mul1, 20 bits at 2 K j for pmcgx pairs, tail-biting);
- pmcgx over all 2^20 states: every masked half is a normal fp16 in [2^-3, 2), and the
  rounding of the exact sums matches torch's float8_e4m3fn cast;
- the FP8 operand of mul1 (2 E4M3(q / 2)) against the same cast.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import codebooks as cb
from workloads import rng_for

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exlr8_codebooks.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        rows.append(line.split())
    return rows


def test_golden_single_states():
    rows = _golden()
    assert len(rows) == 5
    for name, s, a, b in rows:
        s = int(s, 16)
        if name == "mul1":
            assert oracle.mul1_value(s) == int(a)
        else:
            assert oracle.pmcgx_pair_codes(s) == (int(a, 16), int(b, 16))
            v = oracle.pmcgx_values(np.array([int(a, 16), int(b, 16)]))
            assert v[0] == 0.140625 and v[1] == -0.03515625


def test_multipliers_and_ranges():
    assert oracle.MUL1_MULT == 0x83DCD12D
    assert oracle.PMCGX_MULTS == (0xCBAC1FED, 0xBCA14C51)
    q = oracle.mul1_value_array(np.arange(65536))
    assert q.min() >= -510 and q.max() <= 510
    assert np.array_equal(q[[1, 2, 0xFFFF]], [95, -66, -96])


@pytest.mark.parametrize("K", [2, 3, 4])
def test_mul1_scalar_equals_vectorised(K):
    out, inp = 32, 64
    words = rng_for(740, K).integers(0, 2 ** 32, out * inp * K // 32, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(np.array(oracle.decode_unit_mul1_scalar(words, K, out, inp)),
                          oracle.decode_unit_mul1(words, K, out, inp))


@pytest.mark.parametrize("K", [2, 3, 4])
def test_pmcgx_scalar_equals_vectorised(K):
    out, inp = 16, 32
    words = rng_for(741, K).integers(0, 2 ** 32, out * inp * K // 32, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(np.array(oracle.decode_unit_pmcgx_scalar(words, K, out, inp)),
                          oracle.decode_unit_pmcgx(words, K, out, inp))


def _single_bit_tile(K, t):
    words = np.zeros(8 * K, dtype=np.uint32)
    words[t // 32] = np.uint32(1 << (31 - t % 32))
    return words


@pytest.mark.parametrize("K", [2, 3, 4])
def test_window_structure(K):
    nbits = 256 * K
    zero_mul1 = oracle.decode_unit_mul1(np.zeros(8 * K, np.uint32), K, 16, 16)
    zero_pm = oracle.decode_unit_pmcgx(np.zeros(8 * K, np.uint32), K, 16, 16)
    for t in (0, 5, 31, 100, nbits - 17, nbits - 1):
        w = _single_bit_tile(K, t)
        # mul1: position p's state changes iff bit t lies in its window [K p, K p + 16)
        got = oracle.decode_unit_mul1(w, K, 16, 16) != zero_mul1       # [o_l, i_l]
        for p in range(256):
            covers = (t - K * p) % nbits < 16
            if not covers:
                assert not got[p // 16, p % 16]
        # pmcgx: pair j's state changes iff bit t lies in [2 K j, 2 K j + 20); both weights
        # of an untouched pair keep their codes
        gp = oracle.decode_unit_pmcgx(w, K, 16, 16) != zero_pm
        for j in range(128):
            covers = (t - 2 * K * j) % nbits < 20
            for h in (0, 1):
                p = 2 * j + h
                if not covers:
                    assert not gp[p // 16, p % 16]
        states = [s for s in range(256) if (t - K * s) % nbits < 16]
        assert len(states) in (16 // K, 16 // K + 1)


def test_pmcgx_all_states_halves_and_rounding():
    s = np.arange(1 << 20, dtype=np.uint64)
    for c in oracle.PMCGX_MULTS:
        m = (s * np.uint64(c)) & np.uint64(0xFFFFFFFF)
        x = (m & np.uint64(cb.PMCGX_MASK)) ^ np.uint64(cb.PMCGX_XOR)
        halves = []
        for sh in (0, 16):
            h = ((x >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.uint16)
            v = np.abs(oracle.f16_bits_to_f64(h))
            assert np.all((v >= 2.0 ** -3) & (v < 2.0))
            halves.append(oracle.f16_bits_to_f64(h))
        exact = halves[0] + halves[1]
        assert np.all(exact.astype(np.float32).astype(np.float64) == exact)  # exact in fp32
        ref = torch.from_numpy(exact.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = cb._pmcgx_codes_of_states(s.astype(np.int64))[oracle.PMCGX_MULTS.index(c)]
        assert np.array_equal(got, ref)


def test_mul1_fp8_operand():
    q = np.arange(-510, 511)
    got = oracle.mul1_e4m3(q)
    ref = 2.0 * torch.from_numpy((q / 2.0).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.all(np.abs(got - q) <= np.abs(q) * 2.0 ** -4)


@pytest.mark.parametrize("codebook", [1, 2])
def test_pool_contraction_uses_the_codebook(codebook):
    """The parallel oracle's FP8 contraction of a codebook layer equals the plain product of
    the MXFP8 activations with the decoded weights (pmcgx: its E4M3 values; mul1:
    2 E4M3(q / 2)) and the channel scales."""
    from oracle import pool
    rng = rng_for(742, codebook)
    K, E, out, inp = 3, 2, 32, 256
    n = out * inp * K // 32
    lay = {"E": E, "out": out, "in": inp, "layout": 0, "codebook": codebook,
           "bits": np.full(E, K, np.uint8), "code_off": np.arange(E, dtype=np.int64) * n * 4,
           "codes": rng.integers(0, 2 ** 32, E * n, dtype=np.uint64).astype(np.uint32),
           "scales": rng.integers(0x3000, 0x3400, (E, out)).astype(np.uint16),
           "signs": None, "out_signs": None}
    T = 5
    x = oracle.f32_to_bf16_bits_rne(rng.standard_normal((T, inp)).astype(np.float32))
    ids = np.array([[0, 1], [1, 0], [0, -1], [1, 1], [0, 0]], dtype=np.int32)
    y = pool.trellis_slots(lay, x, ids, workers=2, fp8=True)
    xq = oracle.mxfp8_values(oracle.bf16_bits_to_f64(x))
    sc = oracle.f16_bits_to_f64(lay["scales"])
    for e in range(E):
        words = lay["codes"][e * n:(e + 1) * n]
        if codebook == 2:
            w = oracle.pmcgx_values(oracle.decode_unit_pmcgx(words, K, out, inp))
        else:
            w = oracle.mul1_e4m3(oracle.decode_unit_mul1(words, K, out, inp))
        ref = xq @ w.T * sc[e][None, :]
        for t in range(T):
            for k in range(2):
                if ids[t, k] == e:
                    assert np.allclose(y[t, k], ref[t], rtol=1e-12, atol=1e-300)
    assert np.all(y[2, 1] == 0)
