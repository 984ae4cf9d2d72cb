"""Runs the oracle over disjoint sets of experts in spawned worker processes (CPU only).

TEST INFRASTRUCTURE, like the rest of this package: used by the GPU parity tests and by the
benchmark's CPU baseline. It holds none of the method's arithmetic: each worker calls the
oracle's own functions unchanged.

A full-size workload is hundreds of expert units; decoding them one after another takes
minutes in a single process. The outputs of different experts never interact (each
routed slot reads one expert), so the routes are split by expert, each worker calls the
oracle unchanged on the routes of its experts (the other slots masked to -1), and the
parent puts the slots back together. The workers are started with the "spawn" method:
they import numpy and the oracle only, never torch or the GPU library, and read the layer
arrays from shared memory.
"""

import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

from . import (codebooks as _cb, ffn as _ffn, fpbits as _fpbits, gemm as _gemm, hadamard as _had,
               mx as _mx8, mxfp4 as _mx, t16 as _t16)

_ARR = {}
_META = {}
_SHM = []


def _attach(specs, meta):
    # one BLAS thread per worker: the workers already use every core between them
    from threadpoolctl import threadpool_limits
    _SHM.append(threadpool_limits(limits=1))
    for key, (name, shape, dtype) in specs.items():
        shm = shared_memory.SharedMemory(name=name)
        _SHM.append(shm)
        _ARR[key] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)
    _META.update(meta)


def _layer(prefix):
    d = {k: _META[prefix + "." + k] for k in ("E", "out", "in", "layout", "codebook")}
    for k in ("bits", "code_off", "codes", "scales", "signs", "out_signs"):
        d[k] = _ARR.get(prefix + "." + k)
    return d


def _trellis_fns(lay, e4m3=False):
    cache = {}

    def weight_of(e):
        if e not in cache:
            K = int(lay["bits"][e])
            n = lay["out"] * lay["in"] * K // 32
            s = int(lay["code_off"][e]) // 4
            cache.clear()  # one expert at a time: bounded memory
            words = lay["codes"][s:s + n]
            cb = lay["codebook"]
            if cb == 2:    # pmcgx: E4M3 weights by definition (F21)
                cache[e] = _cb.pmcgx_values(_cb.decode_unit_pmcgx(words, K, lay["out"], lay["in"]))
            elif cb == 1:  # mul1 (F20)
                q = _cb.decode_unit_mul1(words, K, lay["out"], lay["in"])
                cache[e] = _cb.mul1_e4m3(q) if e4m3 else q.astype(np.float64)
            else:
                decode = _t16.decode_units128 if lay["layout"] == 2 else _t16.decode_unit
                q = decode(words, K, lay["out"], lay["in"])
                cache[e] = _mx8.t16_e4m3(q) if e4m3 else q.astype(np.float64)
        return cache[e]

    scales = _fpbits.f16_bits_to_f64(lay["scales"])
    return weight_of, (lambda e: scales[e])


def _masked(ids, experts):
    return np.where(np.isin(ids, experts), ids, -1)


def _gemm_task(experts):
    lay = _layer("layer")
    ids = _ARR["ids"]
    gates = _ARR.get("gates")
    keep = _masked(ids, experts)
    flat = np.nonzero(keep.reshape(-1) >= 0)[0]
    if flat.size == 0:
        return flat, np.zeros((0, lay["out"]))
    if _META.get("e4m3"):  # FP8 operands: MXFP8 activation values, E4M3 weights
        y = _gemm.expert_gemm_values(_ARR["x"], keep, gates, lay["E"], *_trellis_fns(lay, True))
    else:
        y = _gemm.expert_gemm(_ARR["x"], keep, gates, lay["E"], *_trellis_fns(lay))
    return flat, y.reshape(-1, lay["out"])[flat]


def _mxfp4_task(experts):
    E, out, inp = _META["mx.E"], _META["mx.out"], _META["mx.in"]
    units = _ARR["mx.units"].reshape(E, -1)
    ids = _ARR["ids"]
    keep = _masked(ids, experts)
    flat = np.nonzero(keep.reshape(-1) >= 0)[0]
    if flat.size == 0:
        return flat, np.zeros((0, out))
    y = _gemm.expert_gemm_values(_ARR["x"], keep, _ARR.get("gates"), E,
                                 lambda e: _mx.decode_mxfp4_unit(units[e], out, inp))
    return flat, y.reshape(-1, out)[flat]


def _ffn_task(experts):
    gu, d = _layer("gate_up"), _layer("down")
    ids = _ARR["ids"]
    keep = _masked(ids, experts)
    if not np.any(keep >= 0):
        return np.zeros((ids.shape[0], d["out"]))
    return _ffn.expert_ffn(_ARR["x"], keep, _ARR.get("gates"), gu["E"], _trellis_fns(gu),
                           _trellis_fns(d), d["signs"], gu["out_signs"], d["out_signs"])


def default_workers():
    """Worker processes: the cores this process may run on, at most 16."""
    return min(16, len(os.sched_getaffinity(0)))


class _Pool:
    def __init__(self, arrays, meta, workers=None):
        n = workers or default_workers()
        self.shms = []
        specs = {}
        for key, a in arrays.items():
            if a is None:
                continue
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            self.shms.append(shm)
            specs[key] = (shm.name, a.shape, a.dtype.str)
        ctx = mp.get_context("spawn")
        self.pool = ctx.Pool(n, initializer=_attach, initargs=(specs, meta))
        self.n = n

    def map(self, fn, items):
        return self.pool.map(fn, items, chunksize=1)

    def close(self):
        self.pool.close()
        self.pool.join()
        for shm in self.shms:
            shm.close()
            shm.unlink()


def _expert_chunks(ids, n, E):
    active = np.unique(ids[(ids >= 0) & (ids < E)])
    k = max(1, min(len(active), 4 * n))
    return [c for c in np.array_split(active, k) if c.size]


def _layer_arrays(prefix, lay):
    arrays = {prefix + "." + k: lay.get(k)
              for k in ("bits", "code_off", "codes", "scales", "signs", "out_signs")}
    meta = {prefix + "." + k: int(lay[k]) for k in ("E", "out", "in")}
    meta[prefix + ".layout"] = int(lay.get("layout", 0))
    meta[prefix + ".codebook"] = int(lay.get("codebook", 0))
    if meta[prefix + ".codebook"] and meta[prefix + ".layout"] == 2:
        raise ValueError("the 128-input unit layout is read for T16 layers only")
    return arrays, meta


def trellis_slots(layer, x_bits, ids, gates=None, workers=None, fp8=False):
    """oracle.expert_gemm of a trellis layer, [T, topk, out], computed expert by expert in
    parallel. Slots with ids outside [0, E) are left as the oracle defines them (0 for -1,
    NaN for invalid ids). With fp8, the FP8 operands of FORMAT F19: the activations' MXFP8
    values (oracle.mxfp8_values of the bf16 x) and the E4M3 roundings of the weights."""
    ids = np.asarray(ids)
    arrays, meta = _layer_arrays("layer", layer)
    if fp8:
        x_bits = _mx8.mxfp8_values(_fpbits.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)))
        meta["e4m3"] = 1
    arrays.update({"x": x_bits, "ids": ids, "gates": gates})
    pool = _Pool(arrays, meta, workers)
    try:
        parts = pool.map(_gemm_task, _expert_chunks(ids, pool.n, layer["E"]))
    finally:
        pool.close()
    y = np.zeros((ids.size, layer["out"]))
    for flat, rows in parts:
        y[flat] = rows
    if layer.get("out_signs") is not None:  # the output-side rotation (FORMAT F17)
        y = _had.output_rotation128(y, layer["out_signs"])
    bad = ((ids < -1) | (ids >= layer["E"])).reshape(-1)
    y[bad] = np.nan
    return y.reshape(ids.shape + (layer["out"],))


def ffn(gate_up, down, x_rot_bits, ids, gates=None, workers=None):
    """oracle.expert_ffn, [T, H], summed over disjoint expert sets computed in parallel."""
    ids = np.asarray(ids)
    arrays, meta = {}, {}
    for p, lay in (("gate_up", gate_up), ("down", down)):
        a, m = _layer_arrays(p, lay)
        arrays.update(a)
        meta.update(m)
    arrays.update({"x": x_rot_bits, "ids": ids, "gates": gates})
    pool = _Pool(arrays, meta, workers)
    try:
        parts = pool.map(_ffn_task, _expert_chunks(ids, pool.n, gate_up["E"]))
    finally:
        pool.close()
    y = np.sum(parts, axis=0)
    y[np.any((ids < -1) | (ids >= gate_up["E"]), axis=1)] = np.nan  # as the oracle: NaN rows
    return y


def mxfp4_slots(layer, x_vals, ids, gates=None, workers=None):
    """oracle.expert_gemm_values of an MXFP4 layer over FP64 activation values, [T, topk,
    out], computed expert by expert in parallel (0 for -1 slots, NaN for invalid ids)."""
    ids = np.asarray(ids)
    arrays = {"mx.units": layer["units"], "x": np.asarray(x_vals, dtype=np.float64),
              "ids": ids, "gates": gates}
    meta = {"mx.E": int(layer["E"]), "mx.out": int(layer["out"]), "mx.in": int(layer["in"])}
    pool = _Pool(arrays, meta, workers)
    try:
        parts = pool.map(_mxfp4_task, _expert_chunks(ids, pool.n, layer["E"]))
    finally:
        pool.close()
    y = np.zeros((ids.size, layer["out"]))
    for flat, rows in parts:
        y[flat] = rows
    y[((ids < -1) | (ids >= layer["E"])).reshape(-1)] = np.nan
    return y.reshape(ids.shape + (layer["out"],))
