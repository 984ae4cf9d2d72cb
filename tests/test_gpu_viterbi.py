"""Encode, then decode on the GPU: Gaussian weights encoded by the oracle's tail-biting
Viterbi search (T16 codebook) come back from the device decoders (decode hook paths 0 and 1)
as exactly the values the search chose, and the trellis GEMM over the encoded unit equals
the FP64 product with that reconstruction (relative L2 <= 1e-3)."""

import numpy as np
import pytest

import oracle
from oracle import viterbi as vt
from gpu_helpers import gpu, needs_gpu, ops, rel_l2, to_dev, torch
from workloads import bf16_from_normal, rng_for

pytestmark = [gpu, needs_gpu]


@pytest.mark.parametrize("K", [2, 3, 4])
def test_viterbi_round_trip_through_gpu_decoders(K):
    o = ops()
    values = oracle.t16_value_array(np.arange(65536)).astype(np.float64)
    out, inp = 16, 256
    W = rng_for(870, K).standard_normal((out, inp))
    scale = 1.0 / values.std()
    words, recon, _ = vt.encode_unit(W, K, values, scale)
    q_ref = np.rint(recon / scale).astype(np.int64)
    for path in (0, 1):
        q = o.trellis_decode(to_dev(words, np.int32), K, out, inp, path).cpu().numpy()
        assert np.array_equal(q.astype(np.int64), q_ref)
    s16 = np.float16(scale).view(np.uint16)
    layer = {"E": 1, "out": out, "in": inp, "bits": np.array([K], np.uint8),
             "code_off": np.zeros(1, np.int64), "codes": words,
             "scales": np.full((1, out), s16, np.uint16), "signs": None}
    T = 24
    x = bf16_from_normal(rng_for(870, K, 1), (T, inp))
    ids = np.zeros((T, 1), np.int32)
    L = o.TrellisLayer.from_host(layer)
    for flags in (o.TQ_GEMV, o.TQ_GEMM):
        y = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), flags=flags)
        torch.cuda.synchronize()
        ref = oracle.bf16_bits_to_f64(x) @ (q_ref * float(np.float16(scale))).T
        assert rel_l2(y.cpu().numpy().reshape(T, out), ref) <= 1e-3
