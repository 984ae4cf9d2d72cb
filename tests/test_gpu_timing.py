"""The measurement hook tq_time_kernel (test infrastructure of the benchmark): the event
pair it is given covers the call's main kernel (a positive interval no longer than the
whole call), it changes no result bit, one call consumes it, and it works under graph
capture and for a launch whose workgroups find no work."""

import time

import numpy as np
import pytest

from gpu_helpers import dev, gpu, needs_gpu, ops, to_dev, torch
from workloads import bf16_from_normal, mxfp4_layer, rng_for, trellis_layer, uniform_routes

pytestmark = [gpu, needs_gpu]


def _events():
    """A timing event pair, each recorded once (torch computes an elapsed time only between
    events it has seen recorded; the hook then sets them again)."""
    e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for ev in e:
        ev.record()
    torch.cuda.synchronize()
    return e


def _trellis(seed, E=12, T=40, topk=4, out=128, inp=512):
    o = ops()
    widths = rng_for(seed, 9).integers(2, 5, size=E).astype(np.uint8)
    L = o.TrellisLayer.from_host(trellis_layer(seed, widths, out, inp, with_signs=True))
    x = to_dev(bf16_from_normal(rng_for(seed, 1), (T, inp)), np.int16)
    ids = to_dev(uniform_routes(rng_for(seed, 2), T, E, topk))
    return L, x, ids


@pytest.mark.parametrize("mode", ["GEMV", "GEMM"])
def test_trellis_kernel_interval(mode):
    o = ops()
    flags = getattr(o, "TQ_" + mode)
    L, x, ids = _trellis(950)
    plain = o.trellis_expert_gemm(L, x, ids, flags=flags).cpu().numpy()
    e0, e1 = _events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o.time_kernel(e0, e1)
    y = o.trellis_expert_gemm(L, x, ids, flags=flags)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms <= wall_ms, (ms, wall_ms)
    assert np.array_equal(y.cpu().numpy(), plain)
    # the hook is consumed: a further call leaves the events as they were
    o.trellis_expert_gemm(L, x, ids, flags=flags)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms


def test_mxfp4_kernel_interval():
    o = ops()
    E, T, topk = 7, 33, 3
    L = o.Mxfp4Layer.from_host(mxfp4_layer(951, E, 256, 1024))
    x = to_dev(bf16_from_normal(rng_for(951, 1), (T, 1024)), np.int16)
    ids = to_dev(uniform_routes(rng_for(951, 2), T, E, topk))
    for flags in (o.TQ_GEMV, o.TQ_GEMM):
        plain = o.mxfp4_expert_gemm(L, x, ids, flags=flags).cpu().numpy()
        e0, e1 = _events()
        o.time_kernel(e0, e1)
        y = o.mxfp4_expert_gemm(L, x, ids, flags=flags)
        torch.cuda.synchronize()
        assert e0.elapsed_time(e1) > 0.0
        assert np.array_equal(y.cpu().numpy(), plain)


def test_interval_under_graph_capture():
    """Under capture the events are recorded around the launch: each replay sets them."""
    o = ops()
    T, topk = 40, 4
    L, x, ids = _trellis(952, T=T, topk=topk)
    ws = o.workspace(T, topk, 12, 128, 512, o.TQ_GEMV)
    y = torch.empty((T, topk, 128), dtype=torch.float32, device=dev())
    o.trellis_expert_gemm(L, x, ids, flags=o.TQ_GEMV, out=y, ws=ws)
    torch.cuda.synchronize()
    plain = y.cpu().numpy()
    e0, e1 = _events()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o.time_kernel(e0, e1)
        o.trellis_expert_gemm(L, x, ids, flags=o.TQ_GEMV, out=y, ws=ws)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert e0.elapsed_time(e1) > 0.0
        assert np.array_equal(y.cpu().numpy(), plain)


def test_interval_of_a_launch_with_no_items():
    """Every route empty: the prefill GEMM's workgroups find no work item and leave; the
    interval is short and the outputs are zero."""
    o = ops()
    L, x, ids = _trellis(953)
    ids.fill_(-1)
    e0, e1 = _events()
    o.time_kernel(e0, e1)
    y = o.trellis_expert_gemm(L, x, ids, flags=o.TQ_GEMM)
    torch.cuda.synchronize()
    assert 0.0 <= e0.elapsed_time(e1) < 1.0
    assert np.all(y.cpu().numpy() == 0)
