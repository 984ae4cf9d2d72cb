"""Helpers for the GPU parity tests: upload seeded workloads, run the oracle on the same
inputs, compare. The oracle never sees a value the GPU produced except where a test
compares two GPU results with each other."""

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

gpu = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def ops():
    from trellis_quantized_moe_amd import ops as _ops
    return _ops


def dev():
    return torch.device("cuda", 0)


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = a.view(dtype)
    return torch.from_numpy(a).to(dev())


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def slot_errors(got, ref):
    """(pooled relative L2, largest per-slot relative L2) over the last axis. A slot whose
    reference is all zero must be all zero (its error is then 0, else inf)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    per = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return rel_l2(got, ref), float(per.max())


def trellis_weight_fns(layer):
    """weight_of / scale_of for the oracle contraction of a host trellis layer."""
    cache = {}

    def weight_of(e):
        if e not in cache:
            K = int(layer["bits"][e])
            nwords = layer["out"] * layer["in"] * K // 32
            start = int(layer["code_off"][e]) // 4
            decode = oracle.decode_units128 if layer.get("layout", 0) == 2 else oracle.decode_unit
            cache[e] = decode(layer["codes"][start:start + nwords], K,
                              layer["out"], layer["in"]).astype(np.float64)
        return cache[e]

    scales = oracle.f16_bits_to_f64(layer["scales"])

    def scale_of(e):
        return scales[e]

    return weight_of, scale_of


def mxfp4_weight_fn(layer):
    ub = oracle.mxfp4_unit_bytes(layer["out"], layer["in"])
    units = layer["units"].reshape(layer["E"], ub)
    return lambda e: oracle.decode_mxfp4_unit(units[e], layer["out"], layer["in"])


def oracle_trellis(layer, x_rot_bits, ids, gates, sample=None):
    """FP64 oracle outputs [T, topk, out]; with `sample` (flat slot indices) only those
    slots are computed (others are zero)."""
    ids = np.asarray(ids)
    if sample is not None:
        keep = np.full(ids.size, -1, dtype=np.int64)
        keep[sample] = ids.reshape(-1)[sample]
        ids = keep.reshape(ids.shape)
    w, s = trellis_weight_fns(layer)
    y = oracle.expert_gemm(x_rot_bits, ids, gates, layer["E"], w, s)
    if layer.get("out_signs") is not None:  # the output-side rotation (FORMAT F17)
        y = oracle.output_rotation128(y, layer["out_signs"])
    return y


def oracle_mxfp4(layer, x_bits, ids, gates, sample=None):
    ids = np.asarray(ids)
    if sample is not None:
        keep = np.full(ids.size, -1, dtype=np.int64)
        keep[sample] = ids.reshape(-1)[sample]
        ids = keep.reshape(ids.shape)
    return oracle.expert_gemm(x_bits, ids, gates, layer["E"], mxfp4_weight_fn(layer), None)


def rotate_host(wl):
    """x~ for a workload: the oracle's fp32-order rotation (FORMAT F8) when it rotates."""
    if not wl["rotate"]:
        return wl["x"]
    return oracle.hadamard128_fp32_order(wl["x"], wl["layer"]["signs"])
