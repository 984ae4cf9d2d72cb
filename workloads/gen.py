"""Seeded input generators (see the package docstring for the recipe)."""

import numpy as np

__all__ = [
    "rng_for", "bf16_from_normal", "fp16_scales", "random_words", "random_signs",
    "uniform_routes", "zipf_routes", "softmax_gates", "trellis_layer", "mxfp4_layer",
    "single_matrix", "one_unit", "mxfp4_decode_layer", "mixed_widths", "mixed_layer",
    "prefill_chunk", "mxfp4_prefill_chunk", "ffn_layers", "ffn_decode", "fp8b32_layer",
    "shared_expert",
    "WORKLOADS",
]

CODES, SCALES, SIGNS, ACTS, ROUTES, GATES, WIDTHS = range(7)


def rng_for(workload, tensor, *extra):
    return np.random.default_rng([int(workload), int(tensor)] + [int(v) for v in extra])


def bf16_from_normal(rng, shape):
    """N(0, 1) drawn in fp32, rounded to bf16 nearest-even; returns uint16 patterns."""
    f = rng.standard_normal(shape, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def fp16_scales(rng, shape, inputs):
    """U(0.5, 1.5) / sqrt(inputs), rounded to fp16; returns uint16 patterns."""
    v = rng.uniform(0.5, 1.5, size=shape) / np.sqrt(float(inputs))
    return v.astype(np.float16).view(np.uint16)


def random_words(rng, n):
    """n uniform uint32 words."""
    return rng.integers(0, 1 << 32, size=int(n), dtype=np.uint32)


def random_signs(rng, n):
    return np.where(rng.integers(0, 2, size=n) == 1, 1, -1).astype(np.int8)


def uniform_routes(rng, T, E, topk):
    """topk distinct experts per token, uniformly at random (int32 [T, topk])."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :topk].astype(np.int32)


def zipf_routes(rng, T, E, topk, s=1.1):
    """topk distinct experts per token, drawn without replacement in proportion to a
    Zipf(s) popularity over a seeded permutation of the expert ids (Gumbel top-k)."""
    perm = rng.permutation(E)
    pop = np.empty(E)
    pop[perm] = 1.0 / np.arange(1, E + 1) ** s
    logp = np.log(pop / pop.sum())
    ids = np.empty((T, topk), dtype=np.int32)
    chunk = 1024
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        g = rng.gumbel(size=(t1 - t0, E))
        ids[t0:t1] = np.argsort(-(logp[None, :] + g), axis=1)[:, :topk]
    return ids


def softmax_gates(rng, T, topk):
    z = rng.standard_normal((T, topk))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def trellis_layer(workload, widths, out, inputs, with_signs, extra=()):
    """A trellis expert layer: one unit per expert, grouped by width (k2, k3, k4), each
    group in ascending expert id; every unit's words drawn uniformly."""
    widths = np.asarray(widths, dtype=np.uint8)
    E = widths.size
    unit_words = {K: out * inputs * K // 32 for K in (2, 3, 4)}
    order = [e for K in (2, 3, 4) for e in range(E) if widths[e] == K]
    code_off = np.zeros(E, dtype=np.int64)
    pos = 0
    for e in order:
        code_off[e] = pos * 4
        pos += unit_words[int(widths[e])]
    codes = random_words(rng_for(workload, CODES, *extra), pos)
    scales = fp16_scales(rng_for(workload, SCALES, *extra), (E, out), inputs)
    signs = random_signs(rng_for(workload, SIGNS, *extra), inputs) if with_signs else None
    return {"E": E, "out": out, "in": inputs, "bits": widths, "code_off": code_off,
            "codes": codes, "scales": scales, "signs": signs}


def mxfp4_layer(workload, E, out, inputs, extra=()):
    """E MXFP4 units (codes uint8 [out][in/2], then E8M0 bytes [out][in/32]) back to back."""
    rng = rng_for(workload, CODES, *extra)
    nc, ns = out * inputs // 2, out * inputs // 32
    units = np.empty((E, nc + ns), dtype=np.uint8)
    units[:, :nc] = rng.integers(0, 256, size=(E, nc), dtype=np.uint8)
    units[:, nc:] = rng_for(workload, SCALES, *extra).integers(119, 126, size=(E, ns), dtype=np.uint8)
    return {"E": E, "out": out, "in": inputs, "units": units.reshape(-1)}


# ----------------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------------

def single_matrix():
    """256 x 256 at K = 2, one bf16 vector, no rotation (the small correctness case)."""
    layer = trellis_layer(1, [2], 256, 256, with_signs=False)
    x = bf16_from_normal(rng_for(1, ACTS), (1, 256))
    ids = np.zeros((1, 1), dtype=np.int32)
    return {"name": "single_256x256_k2", "kind": "trellis", "layer": layer, "x": x,
            "topk_ids": ids, "topk_w": None, "rotate": False}


def one_unit(K, T):
    """One 128 x 5120 unit at width K, 128-wide rotation with random signs, T tokens."""
    layer = trellis_layer(2, [K], 128, 5120, with_signs=True, extra=(K, T))
    x = bf16_from_normal(rng_for(2, ACTS, K, T), (T, 5120))
    ids = np.zeros((T, 1), dtype=np.int32)
    return {"name": "unit_k%d_t%d" % (K, T), "kind": "trellis", "layer": layer, "x": x,
            "topk_ids": ids, "topk_w": None, "rotate": True}


def mxfp4_decode_layer(E=384, T=64, topk=8):
    """MXFP4 routed layer: E units of 128 x 5120, T tokens, top-k uniform, softmax gates."""
    layer = mxfp4_layer(3, E, 128, 5120)
    x = bf16_from_normal(rng_for(3, ACTS), (T, 5120))
    ids = uniform_routes(rng_for(3, ROUTES), T, E, topk)
    w = softmax_gates(rng_for(3, GATES), T, topk)
    return {"name": "mxfp4_e%d_t%d_top%d" % (E, T, topk), "kind": "mxfp4", "layer": layer,
            "x": x, "topk_ids": ids, "topk_w": w, "rotate": False}


def mxfp4_prefill_chunk(E=384, T=8192, topk=8):
    """MXFP4 prefill chunk: the MXFP4 layer's shapes (384 units of 128 x 5120), T tokens
    routed top-k by Zipf(1.1) popularity as the trellis prefill chunk, softmax gates."""
    layer = mxfp4_layer(9, E, 128, 5120)
    x = bf16_from_normal(rng_for(9, ACTS), (T, 5120))
    ids = zipf_routes(rng_for(9, ROUTES), T, E, topk)
    w = softmax_gates(rng_for(9, GATES), T, topk)
    return {"name": "mxfp4_prefill_e%d_t%d_top%d" % (E, T, topk), "kind": "mxfp4",
            "layer": layer, "x": x, "topk_ids": ids, "topk_w": w, "rotate": False}


def fp8b32_layer(workload, E, out, inputs, extra=()):
    """E fp8b32 units (codes uint8 [out][in], then E8M0 bytes [out/32][in/32]) back to back.
    Codes are uniform over the 254 non-NaN E4M3 bytes, scale bytes uniform in 113..119
    (exponents -14..-8)."""
    rng = rng_for(workload, CODES, *extra)
    nc, ns = out * inputs, (out // 32) * (inputs // 32)
    units = np.empty((E, nc + ns), dtype=np.uint8)
    c = rng.integers(0, 254, size=(E, nc), dtype=np.uint8)
    units[:, :nc] = c + (c >= 0x7F) + (c >= 0xFE)  # skip 0x7F and 0xFF (NaN)
    units[:, nc:] = rng_for(workload, SCALES, *extra).integers(113, 120, size=(E, ns), dtype=np.uint8)
    return {"E": E, "out": out, "in": inputs, "units": units.reshape(-1)}


def shared_expert(T=128, out=1536, inputs=5120):
    """The shared expert's gate and up projections (2 x 768 channels over 5120 inputs) in the
    fp8b32 store: one expert that every token routes to."""
    layer = fp8b32_layer(8, 1, out, inputs)
    x = bf16_from_normal(rng_for(8, ACTS), (T, inputs))
    ids = np.zeros((T, 1), dtype=np.int32)
    return {"name": "shared_fp8b32_t%d_%dx%d" % (T, out, inputs), "kind": "fp8b32",
            "layer": layer, "x": x, "topk_ids": ids, "topk_w": None, "rotate": False}


def mixed_widths(E=384, n3=15, n4=1):
    perm = rng_for(4, WIDTHS).permutation(E)
    widths = np.full(E, 2, dtype=np.uint8)
    widths[perm[:n3]] = 3
    widths[perm[n3:n3 + n4]] = 4
    return widths


def mixed_layer(E=384, T=128, topk=8):
    """Mixed-width trellis layer: 368 K=2, 15 K=3, 1 K=4 experts of 128 x 5120 (the
    page's 608 and 21 wider experts out of 15,360, scaled to 384), T tokens, top-k
    uniform, rotated inputs."""
    n3 = round(E * 608 / 15360)
    n4 = max(1, round(E * 21 / 15360))
    layer = trellis_layer(4, mixed_widths(E, n3, n4), 128, 5120, with_signs=True)
    x = bf16_from_normal(rng_for(4, ACTS), (T, 5120))
    ids = uniform_routes(rng_for(4, ROUTES), T, E, topk)
    return {"name": "mixed_e%d_t%d_top%d" % (E, T, topk), "kind": "trellis", "layer": layer,
            "x": x, "topk_ids": ids, "topk_w": None, "rotate": True}


def prefill_chunk(E=384, T=8192, topk=8, K=3):
    """Prefill chunk: T tokens, top-k over E K=3 experts with Zipf(1.1) popularity."""
    layer = trellis_layer(5, np.full(E, K, dtype=np.uint8), 128, 5120, with_signs=True)
    x = bf16_from_normal(rng_for(5, ACTS), (T, 5120))
    ids = zipf_routes(rng_for(5, ROUTES), T, E, topk)
    return {"name": "prefill_e%d_t%d_top%d_k%d" % (E, T, topk, K), "kind": "trellis",
            "layer": layer, "x": x, "topk_ids": ids, "topk_w": None, "rotate": True}


def ffn_layers(workload, widths, H, I, extra=(), down_units128=True, out_rotation=False):
    """The fused gate/up layer (2I x H: the gate's I channels, then the up's) and the down
    layer (H x I) of one routed-expert FFN. The gate/up signs rotate the input, the down
    layer's signs the intermediate. The down layer is stored as units of 128 intermediate
    channels (FORMAT F2b, "layout": 2) unless down_units128 is False (one strip-major unit,
    "layout": 0). With out_rotation, both layers also carry output-side signs (FORMAT F17).
    The fp16 scales are U(0.5, 1.5) / (sqrt(in) * 128), so that with N(0, 1) inputs each
    projection's outputs are of order 1 (the decoded integers have a standard deviation of
    about 104)."""
    gate_up = trellis_layer(workload, widths, 2 * I, H, with_signs=True, extra=(0,) + tuple(extra))
    down = trellis_layer(workload, widths, H, I, with_signs=True, extra=(2,) + tuple(extra))
    gate_up["layout"] = 0
    down["layout"] = 2 if down_units128 else 0
    for lay, j in ((gate_up, 0), (down, 2)):
        v = rng_for(workload, SCALES, j, 99, *extra).uniform(0.5, 1.5, size=(lay["E"], lay["out"]))
        lay["scales"] = (v / (np.sqrt(float(lay["in"])) * 128.0)).astype(np.float16).view(np.uint16)
        if out_rotation:
            lay["out_signs"] = random_signs(rng_for(workload, SIGNS, j, 98, *extra), lay["out"])
    return gate_up, down


def ffn_decode(E=384, T=128, topk=8, H=5120, I=768):
    """Routed-expert FFN decode batch: E experts whose gate, up and down projections are
    6 units of 128 intermediate channels each (I = 768, the 18 units per expert of the
    exlr8 layout; gate and up as one 2I-channel layer, down as its 6 units of 128
    intermediate channels), mixed widths as the mixed layer, T tokens, top-k uniform,
    gates."""
    n3 = round(E * 608 / 15360)
    n4 = max(1, round(E * 21 / 15360))
    gate_up, down = ffn_layers(7, mixed_widths(E, n3, n4), H, I)
    x = bf16_from_normal(rng_for(7, ACTS), (T, H))
    ids = uniform_routes(rng_for(7, ROUTES), T, E, topk)
    w = softmax_gates(rng_for(7, GATES), T, topk)
    return {"name": "ffn_e%d_t%d_top%d" % (E, T, topk), "kind": "ffn", "gate_up": gate_up,
            "down": down, "x": x, "topk_ids": ids, "topk_w": w, "rotate": True}


WORKLOADS = {
    "single": single_matrix,
    "unit": one_unit,
    "mxfp4": mxfp4_decode_layer,
    "mixed": mixed_layer,
    "prefill": prefill_chunk,
}
