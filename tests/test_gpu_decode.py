"""GPU decode hooks vs the oracle, bit for bit: the T16 decoders exactly as the decode-batch
(path 0) and prefill (path 1) kernels use them, and the MXFP4 decoder."""

import numpy as np
import pytest

import oracle
from gpu_helpers import dev, gpu, needs_gpu, ops, to_dev
from workloads import mxfp4_layer, random_words, rng_for

pytestmark = [gpu, needs_gpu]


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("shape", [(16, 64), (48, 320), (128, 5120), (256, 256)])
def test_trellis_decode_random(K, path, shape):
    out, inp = shape
    words = random_words(rng_for(200, K, out, inp), out * inp * K // 32)
    q = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, path).cpu().numpy()
    ref = oracle.decode_unit(words, K, out, inp)
    assert np.array_equal(q, ref)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("path", [0, 1])
def test_trellis_decode_special_streams(K, path):
    out, inp = 32, 128
    n = out * inp * K // 32
    tile = np.array([(0x9E3779B9 * (j + 1)) % (1 << 32) for j in range(8 * K)], dtype=np.uint32)
    for words in (np.zeros(n, np.uint32), np.full(n, 0xFFFFFFFF, np.uint32), np.tile(tile, n // tile.size)):
        q = ops().trellis_decode(to_dev(words, np.int32), K, out, inp, path).cpu().numpy()
        assert np.array_equal(q, oracle.decode_unit(words, K, out, inp))


def test_mxfp4_decode_unit():
    lay = mxfp4_layer(201, 1, 128, 5120)
    w = ops().mxfp4_decode(to_dev(lay["units"]), 128, 5120).cpu().numpy().view(np.uint16)
    ref = oracle.f64_to_bf16_bits_exact(oracle.decode_mxfp4_unit(lay["units"], 128, 5120))
    assert np.array_equal(w, ref)


def test_mxfp4_decode_every_code_and_scale():
    # 256 rows: row r uses scale byte r for all its blocks; each row holds all 16 codes.
    out, inp = 256, 64
    codes = np.zeros((out, inp // 2), dtype=np.uint8)
    pattern = np.array([(2 * j) | ((2 * j + 1) << 4) for j in range(8)], dtype=np.uint8)
    codes[:, :8] = pattern[None, :]
    codes[:, 8:16] = pattern[None, ::-1]
    codes[:, 16:] = rng_for(201, 2).integers(0, 256, size=(out, inp // 2 - 16), dtype=np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], inp // 32, axis=1)
    unit = np.concatenate([codes.reshape(-1), scales.reshape(-1)])
    w = ops().mxfp4_decode(to_dev(unit), out, inp).cpu().numpy().view(np.uint16)
    vals = oracle.decode_mxfp4_unit(unit, out, inp)
    nan = np.isnan(vals)
    # scale bytes 253 and 254 push the largest codes past the bf16 range: no exact value
    over = ~nan & (np.abs(np.nan_to_num(vals)) >= 2.0 ** 128)
    assert np.array_equal(np.isnan(oracle.bf16_bits_to_f64(w))[~over], nan[~over])
    ok = ~nan & ~over
    ref = oracle.f64_to_bf16_bits_exact(np.where(ok, vals, 0.0))
    mismatch = np.argwhere((w != ref) & ok)
    assert mismatch.size == 0, (mismatch[:8], w[ok][:4], ref[ok][:4])
