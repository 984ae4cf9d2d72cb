"""trellis_expert_gemm_noalloc (the entry point for callers that cannot allocate: its
workspace is the library's static device scratch) against trellis_expert_gemm with a
workspace of its own: the same kernels, so the same bits. Two calls in a row, the second
smaller, in both modes; a call too large for the scratch is refused before any GPU work."""

import ctypes

import numpy as np
import pytest

from gpu_helpers import gpu, needs_gpu, ops, to_dev, torch
from trellis_quantized_moe_amd import _lib
from workloads import bf16_from_normal, rng_for, softmax_gates, trellis_layer, uniform_routes

pytestmark = [gpu, needs_gpu]


def _layer(seed, E, inp):
    widths = rng_for(seed, 9).integers(2, 5, size=E).astype(np.uint8)
    return trellis_layer(seed, widths, 128, inp, with_signs=True)


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_noalloc_matches_workspace_entry_point(flags):
    o = ops()
    cases = [(940, 48, 64, 8, 2048), (941, 20, 5, 4, 1024)]  # the second call is smaller
    for seed, E, T, topk, inp in cases:
        layer_h = _layer(seed, E, inp)
        L = o.TrellisLayer.from_host(layer_h)
        x = to_dev(bf16_from_normal(rng_for(seed, 1), (T, inp)), np.int16)
        ids_h = uniform_routes(rng_for(seed, 2), T, E, topk)
        ids_h[1, 0] = -1
        ids = to_dev(ids_h)
        gates = to_dev(softmax_gates(rng_for(seed, 3), T, topk))
        for fl in (flags | o.TQ_ROTATE, flags | o.TQ_ROTATE | o.TQ_COMBINE):
            ref = o.trellis_expert_gemm(L, x, ids, gates, flags=fl)
            out = torch.full_like(ref, float("nan"))
            got = o.trellis_expert_gemm_noalloc(L, x, ids, gates, flags=fl, out=out)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (seed, fl)


def test_noalloc_refuses_calls_beyond_the_scratch():
    lib = _lib.load()
    layer = _lib.TrellisLayerC(384, 128, 5120, 0, 0x1000, 0x1000, 0x1000, 0x1000, None, 1 << 30)
    need = lib.tq_workspace_bytes(4096, 8, 384, 128, 5120, 1)
    assert need > _lib.TQ_NOALLOC_SCRATCH_BYTES
    rc = lib.trellis_expert_gemm_noalloc(ctypes.byref(layer), 0x1000, 4096, 0x1000, None, 8,
                                         0x1000, 1, None)
    assert rc == _lib.TQ_EWORKSPACE
    assert b"scratch" in lib.tq_last_error()
