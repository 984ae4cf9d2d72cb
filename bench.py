"""Benchmark of the routed-expert hot path on one MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic input, with
every input already resident in device memory:
  mixed (headline): the mixed-width trellis layer, 384 experts of 128 x 5120 (368 K=2,
      15 K=3, 1 K=4), 128 tokens, top-8 — the plan + activation prep kernel (route scan,
      128-wide signed rotation of the inputs, f16 staging), the decode-batch grouped GEMV
      (fetch, state rebuild, T16 hash, matrix-core contraction) and the piece reduction
      (epilogue);
  mxfp4: the MXFP4 layer, 384 experts, 64 tokens, top-8 with gates — decode-batch GEMV;
  prefill: 8,192 tokens, top-8 over 384 K=3 experts with Zipf(1.1) popularity — the
      activation prep with the fused rotation, route bucketing (three kernels), grouped
      MFMA GEMM;
  nvfp4: the MXFP4 -> NVFP4 transcode of the 384-unit MXFP4 layer (bytes read + written);
  ffn: the routed expert FFN (fused gate/up, SwiGLU, rotated down projection, combine) of
      384 experts with 768 intermediate channels, 128 tokens, top-8 — five launches.
Steps are captured as HIP graphs and replayed; each step reads a different replica of the
code buffer (replicas total >= 1 GiB) so the 256 MB Infinity Cache cannot serve repeats.

value = compressed bytes of the experts a step touches / step time (GB/s), or dense-
equivalent routed flops / step time (TFLOP/s) for prefill. The roofline object times the
dominant kernel (the grouped GEMV) alone: a HIP event pair that its launch
(hipExtLaunchKernel, through tq_time_kernel) sets to the kernel's own start and end on its
stream, over --kernel-iters direct calls of the step's GEMM queued behind a bounded sleep
kernel. Its HBM
traffic comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (bench.py --drive mixed),
calibrated against a plain elementwise copy of known size in the same runs and stored by
bench.py --write-traffic. The CPU baseline times the oracle (test infrastructure) on the
same workload, on every core this process may use.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
MALL_BYTES = 1 << 30          # replicas of the code buffer total at least this much
SLEEP_CYCLES = 60_000_000     # ~25 ms at 2.4 GHz: the GPU is busy while launches queue


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def active_bytes_trellis(layer, ids):
    ids = np.unique(ids[ids >= 0])
    K = layer["bits"][ids].astype(np.int64)
    return int(np.sum(layer["out"] * layer["in"] * K // 8)), len(ids)


def active_bytes_mxfp4(layer, ids):
    ids = np.unique(ids[ids >= 0])
    ub = layer["out"] * layer["in"] // 2 + layer["out"] * layer["in"] // 32
    return int(len(ids) * ub), len(ids)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "trellis_quantized_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_graph_steps(torch, graphs, steps, warmup):
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


GEMV_SOURCES = ["trellis_gemv.hip", "trellis_cols.h", "trellis_decode.h", "gemv_plan.h", "gemv_wave.h",
                "tq_device.h", "tq_internal.h"]


def kernel_events(torch, n):
    """n event pairs for tq_time_kernel; each is recorded once so that it exists."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in starts + stops:
        e.record()
    torch.cuda.synchronize()
    return starts, stops


def time_main_kernel(torch, ops, call, n_replicas, iters):
    """Mean (and median) duration of the main kernel of `call(r)`: direct launches queued
    behind a bounded sleep kernel, each with tq_time_kernel's event pair set to that
    kernel's start and end."""
    starts, stops = kernel_events(torch, iters)
    for r in range(n_replicas):
        call(r)
    torch.cuda.synchronize()
    torch.cuda._sleep(SLEEP_CYCLES)
    for i in range(iters):
        ops.time_kernel(starts[i], stops[i])
        call(i % n_replicas)
    torch.cuda.synchronize()
    return event_means(starts, stops)


def event_means(starts, stops):
    ms = [s.elapsed_time(e) for s, e in zip(starts, stops)]
    return float(np.mean(ms)) / 1e3, float(np.median(ms)) / 1e3


def traffic_from_profile(name, shash, per_launch_algo):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != shash:
        return None
    return int(d["hbm_bytes_per_launch"])


def replicate(torch, t, total_bytes):
    n = max(1, math.ceil(MALL_BYTES / max(1, total_bytes)))
    return [t] + [t.clone() for _ in range(n - 1)]


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------

def bench_mixed(torch, ops, args):
    from workloads import mixed_layer
    wl = mixed_layer()
    lay = wl["layer"]
    dev = torch.device("cuda", 0)
    L = ops.TrellisLayer.from_host(lay, dev).repacked()  # the kernels' read order, once
    x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    T, topk = wl["topk_ids"].shape
    nbytes, n_active = active_bytes_trellis(lay, wl["topk_ids"])
    reps = replicate(torch, L.codes, L.codes.numel() * 4)
    layers = [L.with_codes(c) for c in reps]
    y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
    ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], ops.TQ_AUTO, dev)
    log("mixed: %d active experts, %.1f MB compressed per step, %d replicas"
        % (n_active, nbytes / 1e6, len(reps)))

    def step(r):
        ops.trellis_expert_gemm(layers[r], x, ids, flags=ops.TQ_ROTATE, out=y, ws=ws)

    for r in range(len(reps)):
        step(r)
    torch.cuda.synchronize()
    graphs = []
    for r in range(len(reps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    sec = time_graph_steps(torch, graphs, args.steps, args.warmup)
    kmean, kmed = time_main_kernel(torch, ops, step, len(reps), args.kernel_iters)
    shash = source_hash(GEMV_SOURCES)
    traffic = traffic_from_profile("trellis_gemv_mixed", shash, nbytes)
    return {
        "sec_per_step": sec, "bytes": nbytes, "n_active": n_active,
        "kernel": "trellis_gemv_kernel", "kernel_sec": kmean, "kernel_sec_median": kmed,
        "traffic": traffic, "source_hash": shash,
        "replicas": len(reps), "wl": wl,
    }


def bench_mxfp4(torch, ops, args):
    from workloads import mxfp4_decode_layer
    wl = mxfp4_decode_layer()
    lay = wl["layer"]
    dev = torch.device("cuda", 0)
    L = ops.Mxfp4Layer.from_host(lay, dev).repacked()  # units in the GEMV's read order, once
    x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    gates = torch.from_numpy(wl["topk_w"]).to(dev)
    T, topk = wl["topk_ids"].shape
    nbytes, n_active = active_bytes_mxfp4(lay, wl["topk_ids"])
    reps = replicate(torch, L.units, L.units.numel())
    layers = [L.with_units(u) for u in reps]
    y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
    ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], ops.TQ_AUTO, dev)
    log("mxfp4: %d active experts, %.1f MB per step, %d replicas" % (n_active, nbytes / 1e6, len(reps)))

    def step(r):
        ops.mxfp4_expert_gemm(layers[r], x, ids, gates, out=y, ws=ws)

    for r in range(len(reps)):
        step(r)
    torch.cuda.synchronize()
    graphs = []
    for r in range(len(reps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    sec = time_graph_steps(torch, graphs, args.steps, args.warmup)
    kmean, kmed = time_main_kernel(torch, ops, step, len(reps), args.kernel_iters)
    return {"sec_per_step": sec, "bytes": nbytes, "n_active": n_active,
            "kernel": "mxfp4_gemv_kernel", "kernel_sec": kmean, "kernel_sec_median": kmed}


def bench_nvfp4(torch, ops, args):
    """MXFP4 -> NVFP4 transcode of the 384-unit MXFP4 layer: bytes read (units) + written
    (nibbles, E4M3 scales, fp32 second-level scales, flags) per call."""
    from workloads import mxfp4_decode_layer
    lay = mxfp4_decode_layer()["layer"]
    dev = torch.device("cuda", 0)
    L = ops.Mxfp4Layer.from_host(lay, dev)
    E, out_ch, in_ = lay["E"], lay["out"], lay["in"]
    reps = replicate(torch, L.units, L.units.numel())
    layers = [L.with_units(u) for u in reps]
    outs = []
    for _ in range(2):  # two output sets alternate: together more than the Infinity Cache
        outs.append((torch.empty((E, out_ch * in_ // 2), dtype=torch.uint8, device=dev),
                     torch.empty((E, out_ch, in_ // 16), dtype=torch.uint8, device=dev),
                     torch.empty(E, dtype=torch.float32, device=dev),
                     torch.empty(E, dtype=torch.uint8, device=dev)))
    nbytes = L.units.numel() + sum(t.numel() * t.element_size() for t in outs[0])
    log("nvfp4: %.1f MB per call, %d replicas" % (nbytes / 1e6, len(reps)))

    def step(r):
        ops.mxfp4_to_nvfp4(layers[r], *outs[r % 2])

    for r in range(len(reps)):
        step(r)
    torch.cuda.synchronize()
    graphs = []
    for r in range(len(reps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    steps = max(20, args.steps // 10)
    sec = time_graph_steps(torch, graphs, steps, max(4, args.warmup // 10))
    return {"sec_per_step": sec, "bytes": nbytes, "steps": steps, "kernel": "nvfp4_transcode_kernel"}


def bench_ffn(torch, ops, args):
    """Routed expert FFN decode batch: gate, up, SwiGLU, rotated down projection, combine.
    Bytes = the compressed units (gate + up + down) of the active experts."""
    from workloads import ffn_decode
    wl = ffn_decode()
    dev = torch.device("cuda", 0)
    # both layers repacked once into the kernels' read order
    GU, D = (ops.TrellisLayer.from_host(wl[k], dev).repacked() for k in ("gate_up", "down"))
    x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    gates = torch.from_numpy(wl["topk_w"]).to(dev)
    T, topk = wl["topk_ids"].shape
    nbytes = sum(active_bytes_trellis(wl[k], wl["topk_ids"])[0] for k in ("gate_up", "down"))
    n_active = active_bytes_trellis(wl["gate_up"], wl["topk_ids"])[1]
    E, H, I = GU.E, GU.in_, GU.out // 2
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = ops.ffn_workspace(T, topk, E, H, I, ops.TQ_AUTO, dev)
    log("ffn: %d active experts, %.1f MB compressed per step" % (n_active, nbytes / 1e6))

    def step():
        ops.trellis_expert_ffn(GU, D, x, ids, gates, flags=ops.TQ_ROTATE, out=y, ws=ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    steps = max(20, args.steps // 5)
    sec = time_graph_steps(torch, [g], steps, max(4, args.warmup // 5))
    return {"sec_per_step": sec, "bytes": nbytes, "n_active": n_active, "steps": steps,
            "code_bytes": int(sum(wl[k]["codes"].nbytes for k in ("gate_up", "down")))}


def bench_shared(torch, ops, args):
    """The shared expert's gate and up projections (1536 x 5120) in the fp8b32 store, every
    token routed to it: a 128-token decode batch (unit bytes per step) and an 8,192-token
    prefill chunk (flops per step)."""
    from workloads import shared_expert
    dev = torch.device("cuda", 0)
    res = {}
    for T, key in ((128, "decode"), (8192, "prefill")):
        wl = shared_expert(T=T)
        lay = wl["layer"]
        L = ops.Fp8b32Layer.from_host(lay, dev).repacked()  # the GEMV's read order, once
        x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
        ids = torch.from_numpy(wl["topk_ids"]).to(dev)
        y = torch.empty((T, 1, lay["out"]), dtype=torch.float32, device=dev)
        ws = ops.workspace(T, 1, 1, lay["out"], lay["in"], ops.TQ_AUTO, dev)
        reps = replicate(torch, L.units, L.units.numel()) if key == "decode" else [L.units]
        layers = [L.with_units(u) for u in reps]

        def step(r):
            ops.fp8b32_expert_gemm(layers[r], x, ids, out=y, ws=ws)

        for r in range(len(reps)):
            step(r)
        torch.cuda.synchronize()
        # a step is short next to a graph launch on the host, so each graph holds up to 16
        # consecutive steps (each on its own replica); every step still runs in full
        per = min(16, len(reps))
        graphs = []
        for r0 in range(0, len(reps), per):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(r0, min(len(reps), r0 + per)):
                    step(r)
            graphs.append((g, min(len(reps), r0 + per) - r0))
        steps = args.steps if key == "decode" else max(1, args.steps // 20)
        n_launch = max(1, steps // per)
        for i in range(max(1, min(args.warmup, steps) // per)):
            graphs[i % len(graphs)][0].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        done = 0
        for i in range(n_launch):
            g, k = graphs[i % len(graphs)]
            g.replay()
            done += k
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / done
        steps = done
        kmean, kmed = time_main_kernel(torch, ops, step, len(reps), min(args.kernel_iters, 50))
        res[key] = {"sec_per_step": sec, "kernel_sec": kmean, "steps": steps, "T": T,
                    "bytes": int(L.units.numel()), "flops": 2.0 * T * lay["out"] * lay["in"]}
        log("shared %s: T = %d, %.1f MB of fp8b32 units, %d replicas" % (key, T, L.units.numel() / 1e6, len(reps)))
        del graphs
    return res


def bench_prefill(torch, ops, args, fp8=False):
    """The trellis prefill chunk; with fp8 the FP8 variant (MXFP8 activations x T16 values
    rounded to E4M3 on the block-scaled fp8 matrix cores)."""
    from workloads import prefill_chunk
    wl = prefill_chunk()
    lay = wl["layer"]
    dev = torch.device("cuda", 0)
    L = ops.TrellisLayer.from_host(lay, dev).repacked()  # the kernels' read order, once
    x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    T, topk = wl["topk_ids"].shape
    flops = 2.0 * T * topk * lay["out"] * lay["in"]
    reps = replicate(torch, L.codes, L.codes.numel() * 4)
    layers = [L.with_codes(c) for c in reps]
    y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
    flags = ops.TQ_ROTATE | (ops.TQ_FP8 if fp8 else 0)
    ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], flags, dev)
    log("prefill%s: %.1f GFLOP per step, %d replicas" % (" fp8" if fp8 else "", flops / 1e9,
                                                         len(reps)))

    def step(r):
        ops.trellis_expert_gemm(layers[r], x, ids, flags=flags, out=y, ws=ws)

    for r in range(len(reps)):
        step(r)
    torch.cuda.synchronize()
    graphs = []
    for r in range(len(reps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    steps = max(10, args.steps // 20)
    sec = time_graph_steps(torch, graphs, steps, max(2, args.warmup // 10))
    kmean, kmed = time_main_kernel(torch, ops, step, len(reps), max(10, args.kernel_iters // 10))
    return {"sec_per_step": sec, "flops": flops, "steps": steps,
            "kernel": "tf8_gemm_kernel" if fp8 else "trellis_gemm_kernel", "kernel_sec": kmean,
            "kernel_sec_median": kmed}


def bench_mx_prefill(torch, ops, args):
    """MXFP4 prefill chunk (384 units of 128 x 5120, 8,192 tokens, top-8 Zipf(1.1), gates),
    units repacked once: the bf16 matrix-core GEMM and the FP8 variant (MXFP8 activations x
    the stored E2M1 codes on the block-scaled fp8 x fp4 matrix cores)."""
    from workloads import mxfp4_prefill_chunk
    wl = mxfp4_prefill_chunk()
    lay = wl["layer"]
    dev = torch.device("cuda", 0)
    L = ops.Mxfp4Layer.from_host(lay, dev).repacked()
    x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(wl["topk_ids"]).to(dev)
    gates = torch.from_numpy(wl["topk_w"]).to(dev)
    T, topk = wl["topk_ids"].shape
    flops = 2.0 * T * topk * lay["out"] * lay["in"]
    reps = replicate(torch, L.units, L.units.numel())
    layers = [L.with_units(u) for u in reps]
    y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
    res = {}
    for key, flags in (("bf16", ops.TQ_GEMM), ("fp8", ops.TQ_FP8)):
        ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], flags, dev)

        def step(r):
            ops.mxfp4_expert_gemm(layers[r], x, ids, gates, flags=flags, out=y, ws=ws)

        for r in range(len(reps)):
            step(r)
        torch.cuda.synchronize()
        graphs = []
        for r in range(len(reps)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        steps = max(10, args.steps // 20)
        sec = time_graph_steps(torch, graphs, steps, max(2, args.warmup // 10))
        kmean, kmed = time_main_kernel(torch, ops, step, len(reps), max(10, args.kernel_iters // 10))
        res[key] = {"sec_per_step": sec, "kernel_sec": kmean, "steps": steps, "flops": flops}
        del graphs
    log("mxfp4 prefill: %.1f GFLOP per step, %d replicas" % (flops / 1e9, len(reps)))
    return res


def cpu_baseline_mixed(wl, n_experts):
    """The oracle on a bounded sample, on every core this process may use: rotation of all
    tokens, then decode + FP64 contraction for the slots of n_experts of the active experts
    (0 = all), the experts split among worker processes (oracle.pool), each calling the
    oracle unchanged with one BLAS thread."""
    import oracle
    from oracle import pool
    lay = wl["layer"]
    ids = wl["topk_ids"]
    active = np.unique(ids)
    n = active.size if n_experts <= 0 else min(n_experts, active.size)
    pick = np.random.default_rng(7).choice(active, size=n, replace=False)
    keep = np.where(np.isin(ids, pick), ids, -1)
    nbytes = int(np.sum(lay["out"] * lay["in"] * lay["bits"][pick].astype(np.int64) // 8))
    workers = pool.default_workers()
    t0 = time.perf_counter()
    xr = oracle.hadamard128_fp32_order(wl["x"], lay["signs"])
    pool.trellis_slots(lay, xr, keep, None, workers=workers)
    sec = time.perf_counter() - t0
    return {
        "value": round(nbytes / sec / 1e9, 5), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "sample": "%d of %d active experts of the mixed layer (their %d slots): oracle rotation of "
                  "all 128 tokens + decode + FP64 contraction, %.1f MB compressed, %.1f s wall "
                  "on %d worker processes (worker start-up included)"
                  % (len(pick), active.size, int(np.sum(keep >= 0)), nbytes / 1e6, sec, workers),
    }


# ------------------------------------------------------------------------------------------
# profiler support: a plain workload driver, and the traffic summary of its counter runs
# ------------------------------------------------------------------------------------------

COPY_BYTES = 1 << 30  # the calibration copy reads and writes this many bytes (4x the MALL)


def drive(torch, ops, which, iters):
    """Runs `iters` steps of one workload (no timing), for rocprofv3. The mixed workload
    ends with a calibration copy: torch.bitwise_xor over COPY_BYTES of int32, which reads
    and writes each byte once."""
    from workloads import mixed_layer, mxfp4_decode_layer, prefill_chunk
    dev = torch.device("cuda", 0)
    if which in ("mixed", "prefill", "prefill8"):
        wl = mixed_layer() if which == "mixed" else prefill_chunk()
        lay = wl["layer"]
        L = ops.TrellisLayer.from_host(lay, dev).repacked()
        x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
        ids = torch.from_numpy(wl["topk_ids"]).to(dev)
        T, topk = wl["topk_ids"].shape
        reps = replicate(torch, L.codes, L.codes.numel() * 4)
        layers = [L.with_codes(c) for c in reps]
        y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
        flags = ops.TQ_ROTATE | (ops.TQ_FP8 if which == "prefill8" else 0)
        ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], flags, dev)
        for i in range(iters):
            ops.trellis_expert_gemm(layers[i % len(layers)], x, ids, flags=flags, out=y, ws=ws)
    elif which == "ffn":
        from workloads import ffn_decode
        wl = ffn_decode()
        GU, D = (ops.TrellisLayer.from_host(wl[k], dev).repacked() for k in ("gate_up", "down"))
        x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
        ids = torch.from_numpy(wl["topk_ids"]).to(dev)
        gates = torch.from_numpy(wl["topk_w"]).to(dev)
        T, topk = wl["topk_ids"].shape
        y = torch.empty((T, GU.in_), dtype=torch.float32, device=dev)
        ws = ops.ffn_workspace(T, topk, GU.E, GU.in_, GU.out // 2, ops.TQ_AUTO, dev)
        for i in range(iters):
            ops.trellis_expert_ffn(GU, D, x, ids, gates, flags=ops.TQ_ROTATE, out=y, ws=ws)
    elif which == "shared":
        from workloads import shared_expert
        for T in (128, 8192):
            wl = shared_expert(T=T)
            lay = wl["layer"]
            L = ops.Fp8b32Layer.from_host(lay, dev).repacked()  # the GEMV's read order, once
            x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
            ids = torch.from_numpy(wl["topk_ids"]).to(dev)
            reps = replicate(torch, L.units, L.units.numel()) if T == 128 else [L.units]
            layers = [L.with_units(u) for u in reps]
            y = torch.empty((T, 1, lay["out"]), dtype=torch.float32, device=dev)
            ws = ops.workspace(T, 1, 1, lay["out"], lay["in"], ops.TQ_AUTO, dev)
            for i in range(iters):
                ops.fp8b32_expert_gemm(layers[i % len(layers)], x, ids, out=y, ws=ws)
    elif which == "mxprefill":
        from workloads import mxfp4_prefill_chunk
        wl = mxfp4_prefill_chunk()
        lay = wl["layer"]
        L = ops.Mxfp4Layer.from_host(lay, dev).repacked()
        x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
        ids = torch.from_numpy(wl["topk_ids"]).to(dev)
        gates = torch.from_numpy(wl["topk_w"]).to(dev)
        T, topk = wl["topk_ids"].shape
        reps = replicate(torch, L.units, L.units.numel())
        layers = [L.with_units(u) for u in reps]
        y = torch.empty((T, topk, lay["out"]), dtype=torch.float32, device=dev)
        for flags in (ops.TQ_GEMM, ops.TQ_FP8):
            ws = ops.workspace(T, topk, lay["E"], lay["out"], lay["in"], flags, dev)
            for i in range(iters):
                ops.mxfp4_expert_gemm(layers[i % len(layers)], x, ids, gates, flags=flags, out=y,
                                      ws=ws)
    elif which == "nvfp4":
        lay = mxfp4_decode_layer()["layer"]
        L = ops.Mxfp4Layer.from_host(lay, dev)
        reps = replicate(torch, L.units, L.units.numel())
        layers = [L.with_units(u) for u in reps]
        outs = [ops.mxfp4_to_nvfp4(L) for _ in range(2)]
        for i in range(iters):
            ops.mxfp4_to_nvfp4(layers[i % len(layers)], *outs[i % 2])
    else:
        wl = mxfp4_decode_layer()
        lay = wl["layer"]
        L = ops.Mxfp4Layer.from_host(lay, dev).repacked()
        x = torch.from_numpy(wl["x"].view(np.int16)).to(dev)
        ids = torch.from_numpy(wl["topk_ids"]).to(dev)
        gates = torch.from_numpy(wl["topk_w"]).to(dev)
        reps = replicate(torch, L.units, L.units.numel())
        layers = [L.with_units(u) for u in reps]
        for i in range(iters):
            ops.mxfp4_expert_gemm(layers[i % len(layers)], x, ids, gates)
    if which == "mixed":
        src = torch.arange(COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_xor(src, 0x5A5A5A5A, out=dst)
    torch.cuda.synchronize()
    log("drove %s for %d steps" % (which, iters))


def counter_means(run_dir, counter):
    """Mean value of `counter` per dispatch, by kernel name, from a rocprofv3 csv output."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + run_dir)
    acc = {}
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in acc.items()}


def counter_summary(run_dirs):
    """Per-kernel mean of every counter per dispatch over rocprofv3 csv runs, as a markdown
    table (one row per kernel, one column per counter)."""
    import csv
    import glob
    table, names = {}, []
    for d in run_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under " + d)
        acc = {}
        for r in csv.DictReader(open(files[0])):
            k = _short_kernel_name(r["Kernel_Name"])
            acc.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        for (k, c), v in acc.items():
            if c not in names:
                names.append(c)
            table.setdefault(k, {})[c] = (float(np.mean(v)), len(v))
    print("| kernel | dispatches | " + " | ".join(names) + " |")
    print("|---|---:|" + "---:|" * len(names))
    for k in sorted(table):
        row = table[k]
        n = max(v[1] for v in row.values())
        cells = ["{:,.0f}".format(row[c][0]) if c in row else "" for c in names]
        print("| %s | %d | %s |" % (k, n, " | ".join(cells)))


def _short_kernel_name(name):
    k = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return k.split("(")[0].split("<")[0].strip().split("::")[-1]


def trace_summary(run_dirs):
    """The library's kernels in rocprofv3 --kernel-trace --stats runs (csv output), as a
    markdown table: calls and mean / min / max duration per dispatch."""
    import csv
    import glob
    print("| kernel | calls | mean us | min us | max us |")
    print("|---|---:|---:|---:|---:|")
    for d in run_dirs:
        files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
        if not files:
            raise SystemExit("no kernel_stats.csv under " + d)
        for r in csv.DictReader(open(files[0])):
            if not r["Name"].startswith(("tq::", "void tq::")):
                continue
            print("| %s | %s | %.2f | %.2f | %.2f |" % (
                _short_kernel_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))


def write_traffic(fetch_dir, write_dir, command):
    """HBM bytes per launch of the trellis GEMV from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each divided by what the same counter reads per byte of the calibration copy."""
    fetch = counter_means(fetch_dir, "FETCH_SIZE")
    write = counter_means(write_dir, "WRITE_SIZE")
    pick = lambda d, key: [v for k, v in d.items() if key in k]
    gf, gw = pick(fetch, "trellis_gemv_kernel"), pick(write, "trellis_gemv_kernel")
    cf, cw = pick(fetch, "BitwiseXor"), pick(write, "BitwiseXor")
    if not (gf and gw and cf and cw):
        raise SystemExit("GEMV or calibration-copy dispatches missing in the counter runs")
    f_fac = cf[0] * 1024 / COPY_BYTES
    w_fac = cw[0] * 1024 / COPY_BYTES
    fb, wb = gf[0] * 1024 / f_fac, gw[0] * 1024 / w_fac
    d = {"kernel": "trellis_gemv_kernel", "workload": "mixed",
         "source_hash": source_hash(GEMV_SOURCES),
         "hbm_bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
         "write_bytes": int(round(wb)), "copy_fetch_factor": round(f_fac, 4),
         "copy_write_factor": round(w_fac, 4), "command": command}
    path = os.path.join(ROOT, "profiles", "traffic_trellis_gemv_mixed.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--extras", default="mxfp4,prefill,mxprefill,nvfp4,ffn,shared",
                    help="comma list of secondary workloads (mxfp4, prefill, mxprefill, nvfp4, ffn, "
                         "shared) or 'none'")
    ap.add_argument("--cpu-sample-experts", type=int, default=0,
                    help="active experts in the CPU baseline sample (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--drive", choices=["mixed", "mxfp4", "prefill", "prefill8", "mxprefill",
                                        "nvfp4", "shared", "ffn"],
                    help="only run --steps steps of one workload (for rocprofv3)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs of --drive mixed")
    ap.add_argument("--traffic-command", default="",
                    help="the profiler commands that made the --write-traffic runs")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print per-kernel counter means of rocprofv3 csv runs as markdown")
    ap.add_argument("--trace-summary", nargs="+", metavar="DIR",
                    help="print the library's kernel durations of rocprofv3 csv runs as markdown")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.traffic_command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from trellis_quantized_moe_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.drive:
        drive(torch, ops, args.drive, args.steps)
        return

    res = bench_mixed(torch, ops, args)
    gbs = res["bytes"] / res["sec_per_step"] / 1e9
    achieved = res["bytes"] / res["kernel_sec"] / 1e9
    wl = res.pop("wl")
    line = {
        "metric": "compressed-expert GB/s (decode GEMV) + TFLOP/s (prefill) vs roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["sec_per_step"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "mixed-width trellis layer (K2 Mix style) decode batch",
            "experts": 384, "unit": "128x5120", "widths": "368xK2 15xK3 1xK4",
            "tokens": 128, "topk": 8, "active_experts": res["n_active"],
            "compressed_bytes_per_step": res["bytes"], "rotation": "128-wide signed Hadamard fused into the activation prep",
            "operands": "int8 matrix-core products with int32 sums: the weights' signed bytes, "
                        "activations as 16-bit per-token fixed point in two int8 halves",
            "replicas": res["replicas"],
            "layout": "units repacked once into the kernels' read order (TQ_LAYOUT_GEMV)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": res["traffic"],
            "kernel": res["kernel"],
            "kernel_us": round(res["kernel_sec"] * 1e6, 3),
            "kernel_us_median": round(res["kernel_sec_median"] * 1e6, 3),
            "algorithmic_bytes_per_launch": res["bytes"],
            "source_hash": res["source_hash"],
        },
    }
    extras = {}
    todo = [] if args.extras == "none" else [e for e in args.extras.split(",") if e]
    if "mxfp4" in todo:
        m = bench_mxfp4(torch, ops, args)
        extras["mxfp4_decode_layer"] = {
            "workload": "MXFP4 layer, 384 experts, 64 tokens, top-8, gates",
            "layout": "units repacked once into the GEMV's read order (TQ_LAYOUT_GEMV)",
            "GB/s": round(m["bytes"] / m["sec_per_step"] / 1e9, 2),
            "ms_per_step": round(m["sec_per_step"] * 1e3, 5),
            "kernel": m["kernel"], "kernel_us": round(m["kernel_sec"] * 1e6, 3),
            "kernel_GB/s": round(m["bytes"] / m["kernel_sec"] / 1e9, 2),
            "frac_hbm": round(m["bytes"] / m["kernel_sec"] / 1e9 / HBM_PEAK_GBS, 4),
            "active_experts": m["n_active"], "bytes_per_step": m["bytes"],
        }
    if "prefill" in todo:
        p = bench_prefill(torch, ops, args)
        extras["prefill_chunk"] = {
            "workload": "8192 tokens, top-8, 384 K=3 experts, Zipf(1.1), units repacked once",
            "TFLOP/s": round(p["flops"] / p["sec_per_step"] / 1e12, 3),
            "ms_per_step": round(p["sec_per_step"] * 1e3, 5), "steps": p["steps"],
            "kernel": p["kernel"], "kernel_us": round(p["kernel_sec"] * 1e6, 3),
            "kernel_TFLOP/s": round(p["flops"] / p["kernel_sec"] / 1e12, 3),
            "frac_f16_peak": round(p["flops"] / p["kernel_sec"] / 1e12 / F16_PEAK_TFLOPS, 4),
        }
        f = bench_prefill(torch, ops, args, fp8=True)
        extras["prefill_chunk_fp8"] = {
            "workload": "the same chunk with FP8 operands: MXFP8 activations (rotation fused "
                        "into their prep) x T16 values rounded to E4M3",
            "TFLOP/s": round(f["flops"] / f["sec_per_step"] / 1e12, 3),
            "ms_per_step": round(f["sec_per_step"] * 1e3, 5), "steps": f["steps"],
            "kernel": f["kernel"] + " (v_mfma_scale_f32_16x16x128_f8f6f4, fp8 x fp8)",
            "kernel_us": round(f["kernel_sec"] * 1e6, 3),
            "kernel_TFLOP/s": round(f["flops"] / f["kernel_sec"] / 1e12, 3),
            "frac_fp8_peak": round(f["flops"] / f["kernel_sec"] / 1e12 / FP8_PEAK_TFLOPS, 4),
        }
    if "mxprefill" in todo:
        mp = bench_mx_prefill(torch, ops, args)
        b, f = mp["bf16"], mp["fp8"]
        extras["mxfp4_prefill_chunk"] = {
            "workload": "MXFP4 layer, 384 units of 128 x 5120, 8192 tokens, top-8 Zipf(1.1), gates, "
                        "units repacked once",
            "bf16_TFLOP/s": round(b["flops"] / b["sec_per_step"] / 1e12, 3),
            "bf16_kernel": "mxfp4_prefill_kernel", "bf16_kernel_us": round(b["kernel_sec"] * 1e6, 3),
            "bf16_frac_bf16_peak": round(b["flops"] / b["kernel_sec"] / 1e12 / F16_PEAK_TFLOPS, 4),
            "fp8_TFLOP/s": round(f["flops"] / f["sec_per_step"] / 1e12, 3),
            "fp8_ms_per_step": round(f["sec_per_step"] * 1e3, 5),
            "fp8_kernel": "mx8_gemm_kernel (MXFP8 x MXFP4, v_mfma_scale_f32_16x16x128_f8f6f4)",
            "fp8_kernel_us": round(f["kernel_sec"] * 1e6, 3),
            "fp8_kernel_TFLOP/s": round(f["flops"] / f["kernel_sec"] / 1e12, 3),
            "fp8_frac_fp8_peak": round(f["flops"] / f["kernel_sec"] / 1e12 / FP8_PEAK_TFLOPS, 4),
        }
    if "nvfp4" in todo:
        v = bench_nvfp4(torch, ops, args)
        extras["nvfp4_transcode"] = {
            "workload": "MXFP4 -> NVFP4 transcode of 384 units of 128 x 5120",
            "GB/s": round(v["bytes"] / v["sec_per_step"] / 1e9, 2),
            "us_per_call": round(v["sec_per_step"] * 1e6, 3), "steps": v["steps"],
            "kernel": v["kernel"], "bytes_per_call": v["bytes"],
            "frac_hbm": round(v["bytes"] / v["sec_per_step"] / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "ffn" in todo:
        f = bench_ffn(torch, ops, args)
        extras["ffn_decode"] = {
            "workload": "routed expert FFN, 384 experts (fused gate/up 1536 x 5120, down 5120 x 768 "
                        "in 128-channel units, 368 K2 / 15 K3 / 1 K4), 128 tokens, top-8, gates; "
                        "5 launches (plans + prep, gate/up GEMV, SwiGLU + rotation + down "
                        "operands, down GEMV, reduction + combine), units repacked once",
            "GB/s": round(f["bytes"] / f["sec_per_step"] / 1e9, 2),
            "ms_per_step": round(f["sec_per_step"] * 1e3, 5), "steps": f["steps"],
            "active_experts": f["n_active"], "compressed_bytes_per_step": f["bytes"],
            "frac_hbm": round(f["bytes"] / f["sec_per_step"] / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "shared" in todo:
        sh = bench_shared(torch, ops, args)
        d, pf = sh["decode"], sh["prefill"]
        extras["shared_expert_fp8b32"] = {
            "workload": "shared expert gate+up (1536 x 5120, fp8b32: E4M3, E8M0 per 32 x 32 block), "
                        "every token routed to it",
            "layout": "unit repacked once into the GEMV's read order (TQ_LAYOUT_GEMV)",
            "decode_tokens": d["T"], "decode_GB/s": round(d["bytes"] / d["sec_per_step"] / 1e9, 2),
            "decode_us_per_step": round(d["sec_per_step"] * 1e6, 3),
            "decode_kernel": "mxfp4_gemv_kernel<fp8b32>",
            "decode_kernel_us": round(d["kernel_sec"] * 1e6, 3),
            "decode_frac_hbm": round(d["bytes"] / d["kernel_sec"] / 1e9 / HBM_PEAK_GBS, 4),
            "unit_bytes": d["bytes"],
            "prefill_tokens": pf["T"], "prefill_TFLOP/s": round(pf["flops"] / pf["sec_per_step"] / 1e12, 3),
            "prefill_ms_per_step": round(pf["sec_per_step"] * 1e3, 5),
            "prefill_kernel": "mxfp4_prefill_kernel<fp8b32>",
            "prefill_kernel_us": round(pf["kernel_sec"] * 1e6, 3),
            "prefill_frac_bf16_peak": round(pf["flops"] / pf["kernel_sec"] / 1e12 / F16_PEAK_TFLOPS, 4),
        }
    if extras:
        line["extras"] = extras
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_mixed(wl, args.cpu_sample_experts)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
