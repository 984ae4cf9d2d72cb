"""Trellis expert GEMV / GEMM on the GPU vs the FP64 oracle (relative L2 <= 1e-3, the bound
the FORMAT note fixes), plus the structural invariants: determinism, token permutation,
mixed width == single width, empty and invalid slots, combine, graph replay."""

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from gpu_helpers import (dev, gpu, needs_gpu, ops, oracle_trellis, rel_l2, rotate_host,
                         slot_errors, to_dev, torch)
from workloads import (bf16_from_normal, mixed_layer, one_unit, prefill_chunk, rng_for,
                       single_matrix, softmax_gates, trellis_layer, uniform_routes, zipf_routes)

pytestmark = [gpu, needs_gpu]
TOL = 1e-3


def run(layer_h, x_bits, ids, gates=None, flags=0, rotate_signs=None):
    o = ops()
    L = o.TrellisLayer.from_host(layer_h)
    x = to_dev(x_bits, np.int16)
    if rotate_signs is not None:
        x = o.hadamard128(x, to_dev(rotate_signs))
    y = o.trellis_expert_gemm(L, x, to_dev(ids), None if gates is None else to_dev(gates),
                              flags=flags)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def small_layer(seed, E, out, inp, widths=None):
    w = np.asarray(widths if widths is not None else rng_for(seed, 9).integers(2, 5, size=E),
                   dtype=np.uint8)
    return trellis_layer(seed, w, out, inp, with_signs=True)


def test_single_matrix_256():
    wl = single_matrix()
    y = run(wl["layer"], wl["x"], wl["topk_ids"])
    ref = oracle_trellis(wl["layer"], wl["x"], wl["topk_ids"], None)
    assert rel_l2(y, ref) <= TOL


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("T", [1, 4, 16])
def test_one_unit_rotated(K, T):
    wl = one_unit(K, T)
    y = run(wl["layer"], wl["x"], wl["topk_ids"], rotate_signs=wl["layer"]["signs"])
    ref = oracle_trellis(wl["layer"], rotate_host(wl), wl["topk_ids"], None)
    assert rel_l2(y, ref) <= TOL
    # per output as well: no slot may hide a large error behind the others
    err = np.abs(y - ref).max() / np.abs(ref).max()
    assert err <= 1e-3


@pytest.mark.parametrize("flags", [1, 2])
def test_small_mixed_layer_both_modes(flags):
    E, T, topk = 9, 70, 4
    layer = small_layer(400, E, 128, 1024)
    x = bf16_from_normal(rng_for(400, 1), (T, 1024))
    ids = uniform_routes(rng_for(400, 2), T, E, topk)
    ids[3, 1] = -1
    ids[10, :] = -1
    gates = softmax_gates(rng_for(400, 3), T, topk)
    y = run(layer, x, ids, gates, flags=flags)
    ref = oracle_trellis(layer, x, ids, gates)
    assert rel_l2(y, ref) <= TOL
    assert np.all(y[3, 1] == 0) and np.all(y[10] == 0)


def test_many_tokens_per_expert_in_gemv_mode():
    # more than 16 tokens per expert forces several chunks in the decode-batch kernel
    E, T, topk = 3, 50, 2
    layer = small_layer(401, E, 256, 512, widths=[2, 3, 4])
    x = bf16_from_normal(rng_for(401, 1), (T, 512))
    ids = uniform_routes(rng_for(401, 2), T, E, topk)
    y1 = run(layer, x, ids, flags=1)
    y2 = run(layer, x, ids, flags=2)
    ref = oracle_trellis(layer, x, ids, None)
    assert rel_l2(y1, ref) <= TOL and rel_l2(y2, ref) <= TOL


def test_one_hot_reproduces_decoded_columns():
    layer = small_layer(402, 2, 32, 256, widths=[3, 2])
    x = np.zeros((6, 256), dtype=np.uint16)
    cols = [0, 17, 100, 128, 201, 255]
    for t, c in enumerate(cols):
        x[t, c] = 0x3F80
    ids = np.array([[0], [1], [0], [1], [0], [1]], dtype=np.int32)
    for flags in (1, 2):
        y = run(layer, x, ids, flags=flags)
        sc = oracle.f16_bits_to_f64(layer["scales"]).astype(np.float32)
        for t, c in enumerate(cols):
            e = ids[t, 0]
            K = int(layer["bits"][e])
            nw = 32 * 256 * K // 32
            off = int(layer["code_off"][e]) // 4
            q = oracle.decode_unit(layer["codes"][off:off + nw], K, 32, 256)
            expect = (q[:, c].astype(np.float32) * sc[e]).astype(np.float64)
            assert np.array_equal(y[t, 0], expect), (flags, t)


def test_empty_invalid_and_status():
    o = ops()
    layer = small_layer(403, 4, 128, 512)
    L = o.TrellisLayer.from_host(layer)
    x = to_dev(bf16_from_normal(rng_for(403, 1), (5, 512)), np.int16)
    ids_h = np.array([[0, -1], [7, 1], [2, -5], [3, 3], [-1, -1]], dtype=np.int32)
    for flags in (1, 2):
        ws = o.workspace(5, 2, 4, 128, 512, flags)
        y = o.trellis_expert_gemm(L, x, to_dev(ids_h), flags=flags, ws=ws).cpu().numpy()
        assert np.all(y[0, 1] == 0) and np.all(y[4] == 0)
        assert np.all(np.isnan(y[1, 0])) and np.all(np.isnan(y[2, 1]))
        assert np.all(np.isfinite(y[0, 0])) and np.all(np.isfinite(y[3]))
        assert o.device_status(ws) == 1
        assert o.device_status(ws) == 0


def test_bad_unit_descriptor_gives_nan():
    # a bad width byte (expert 1), a unit reaching past the end of the code buffer (expert
    # 3: its offset is moved up by 16 bytes), a negative offset (expert 4)
    o = ops()
    layer = small_layer(404, 5, 128, 512, widths=[2, 2, 2, 2, 2])
    layer["bits"] = layer["bits"].copy()
    layer["bits"][1] = 5
    layer["code_off"] = layer["code_off"].copy()
    assert layer["code_off"][4] == layer["codes"].nbytes - 128 * 512 * 2 // 8
    layer["code_off"][3] = layer["code_off"][4] + 16
    layer["code_off"][4] = -16
    L = o.TrellisLayer.from_host(layer)
    x = to_dev(bf16_from_normal(rng_for(404, 1), (6, 512)), np.int16)
    ids = to_dev(np.array([[0], [1], [2], [1], [3], [4]], dtype=np.int32))
    for flags in (1, 2):
        ws = o.workspace(6, 1, 5, 128, 512, flags)
        y = o.trellis_expert_gemm(L, x, ids, flags=flags, ws=ws).cpu().numpy()
        for t in (1, 3, 4, 5):
            assert np.all(np.isnan(y[t])), (flags, t)
        assert np.all(np.isfinite(y[0])) and np.all(np.isfinite(y[2]))
        assert o.device_status(ws) == 2


def test_combine_matches_slot_sum():
    E, T, topk = 6, 33, 3
    layer = small_layer(405, E, 128, 512)
    x = bf16_from_normal(rng_for(405, 1), (T, 512))
    ids = uniform_routes(rng_for(405, 2), T, E, topk)
    gates = softmax_gates(rng_for(405, 3), T, topk)
    for flags in (1, 2):
        slots = run(layer, x, ids, gates, flags=flags)
        comb = run(layer, x, ids, gates, flags=flags | 4)
        expect = np.zeros_like(comb)
        for k in range(topk):   # same fp32 additions, same order
            expect = (expect.astype(np.float32) + slots[:, k].astype(np.float32)).astype(np.float64)
        assert np.array_equal(comb, expect)
        ref = oracle.combine_slots(oracle_trellis(layer, x, ids, gates))
        assert rel_l2(comb, ref) <= TOL


def test_deterministic_and_token_permutation():
    E, T, topk = 12, 64, 8
    layer = small_layer(406, E, 128, 1024)
    x = bf16_from_normal(rng_for(406, 1), (T, 1024))
    ids = uniform_routes(rng_for(406, 2), T, E, topk)
    for flags in (1, 2):
        a = run(layer, x, ids, flags=flags)
        b = run(layer, x, ids, flags=flags)
        assert np.array_equal(a, b)
        perm = rng_for(406, 3).permutation(T)
        c = run(layer, x[perm], ids[perm], flags=flags)
        assert np.array_equal(c, a[perm])


def test_mixed_width_matches_single_width_launches():
    E, T, topk = 10, 40, 4
    widths = np.array([2, 3, 4, 2, 2, 3, 4, 2, 3, 2], dtype=np.uint8)
    mixed = small_layer(407, E, 128, 512, widths=widths)
    x = bf16_from_normal(rng_for(407, 1), (T, 512))
    ids = uniform_routes(rng_for(407, 2), T, E, topk)
    for flags in (1, 2):
        y_mixed = run(mixed, x, ids, flags=flags)
        for K in (2, 3, 4):
            # a single-width layer: width-K experts keep their units, the others get fresh
            # width-K units and no routes
            single = small_layer(408 + K, E, 128, 512, widths=np.full(E, K, np.uint8))
            codes = single["codes"].copy()
            for e in range(E):
                if widths[e] == K:
                    n = 128 * 512 * K // 32
                    src = int(mixed["code_off"][e]) // 4
                    dst = int(single["code_off"][e]) // 4
                    codes[dst:dst + n] = mixed["codes"][src:src + n]
            single["codes"] = codes
            single["scales"] = mixed["scales"]
            ids_k = np.where(widths[ids] == K, ids, -1).astype(np.int32)
            y_k = run(single, x, ids_k, flags=flags)
            sel = widths[ids] == K
            # both modes: the decode batch splits an expert's inputs by the whole batch's
            # work, but adds the pieces' exact integer sums, so the split never shows
            assert np.array_equal(y_k[sel], y_mixed[sel]), (flags, K)


def test_decode_batch_slot_bits_do_not_depend_on_the_batch():
    """One token's slots alone, and the same slots inside a large batch over many experts:
    the plan splits the experts' inputs into very different pieces in the two launches (up
    to in / 256 pieces alone, a few inside the large batch), and the results are the
    same bits (FORMAT F14)."""
    E, topk, inp = 64, 8, 5120
    layer = small_layer(416, E, 128, inp)
    x = bf16_from_normal(rng_for(416, 1), (200, inp))
    ids = uniform_routes(rng_for(416, 2), 200, E, topk)
    gates = softmax_gates(rng_for(416, 3), 200, topk)
    big = run(layer, x, ids, gates, flags=1)
    for t in (0, 77, 199):
        alone = run(layer, x[t:t + 1], ids[t:t + 1], gates[t:t + 1], flags=1)
        assert np.array_equal(alone[0], big[t]), t
    ref = oracle_trellis(layer, x, ids, gates)
    assert rel_l2(big, ref) <= TOL


def test_graph_replay_with_changing_routes():
    o = ops()
    E, T, topk = 16, 24, 4
    layer = small_layer(409, E, 128, 512)
    L = o.TrellisLayer.from_host(layer)
    x = to_dev(bf16_from_normal(rng_for(409, 1), (T, 512)), np.int16)
    ids = to_dev(uniform_routes(rng_for(409, 2), T, E, topk))
    for flags in (1, 2):
        ws = o.workspace(T, topk, E, 128, 512, flags)
        y = torch.empty((T, topk, 128), dtype=torch.float32, device=dev())
        o.trellis_expert_gemm(L, x, ids, flags=flags, out=y, ws=ws)  # warm up
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            o.trellis_expert_gemm(L, x, ids, flags=flags, out=y, ws=ws)
        for r in range(3):
            new = uniform_routes(rng_for(409, 10 + r), T, E, topk)
            ids.copy_(to_dev(new))
            g.replay()
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            eager = o.trellis_expert_gemm(L, x, ids, flags=flags).cpu().numpy()
            assert np.array_equal(got, eager), (flags, r)
            ref = oracle_trellis(layer, x.cpu().numpy().view(np.uint16), new, None)
            assert rel_l2(got, ref) <= TOL


@pytest.mark.timeout(900)
def test_mixed_layer_full_size_every_slot():
    """The mixed-width decode batch at full size (384 experts of 128 x 5120, 368 K=2, 15
    K=3, 1 K=4, 128 tokens, top-8, the rotation fused), every one of the 1,024 slots
    against the FP64 oracle: pooled and per-slot relative L2."""
    wl = mixed_layer()
    layer = wl["layer"]
    o = ops()
    L = o.TrellisLayer.from_host(layer)
    y = o.trellis_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                              flags=o.TQ_ROTATE)
    y = y.cpu().numpy()
    ref = oracle_pool.trellis_slots(layer, rotate_host(wl), wl["topk_ids"])
    pooled, worst = slot_errors(y, ref)
    print("mixed layer, 1024 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL


@pytest.mark.timeout(900)
def test_prefill_chunk_full_size_every_slot():
    """The prefill chunk at full size (8,192 tokens, top-8, 384 K=3 experts, Zipf(1.1)
    popularity, the rotation fused), every one of the 65,536 slots against the FP64
    oracle: pooled and per-slot relative L2."""
    wl = prefill_chunk()
    layer = wl["layer"]
    o = ops()
    L = o.TrellisLayer.from_host(layer)
    y = o.trellis_expert_gemm(L, to_dev(wl["x"], np.int16), to_dev(wl["topk_ids"]),
                              flags=o.TQ_ROTATE)
    y = y.cpu().numpy()
    ref = oracle_pool.trellis_slots(layer, rotate_host(wl), wl["topk_ids"])
    pooled, worst = slot_errors(y, ref)
    print("prefill chunk, 65536 slots: pooled %.3e, worst slot %.3e" % (pooled, worst))
    assert pooled <= TOL and worst <= TOL


@pytest.mark.parametrize("flags", [1, 2])
def test_fused_rotation_equals_separate_hadamard(flags):
    """TQ_ROTATE applies the layer's signed 128-wide rotation inside the activation prep:
    the result is bit-identical to rotating first with hadamard128 (same fp32 butterfly,
    same bf16 rounding) and calling without the flag."""
    o = ops()
    E, T, topk, inp = 12, 37, 4, 768
    layer = small_layer(412, E, 256, inp)
    L = o.TrellisLayer.from_host(layer)
    x = to_dev(bf16_from_normal(rng_for(412, 1), (T, inp)), np.int16)
    ids = to_dev(uniform_routes(rng_for(412, 2), T, E, topk))
    gates = to_dev(softmax_gates(rng_for(412, 3), T, topk))
    fused = o.trellis_expert_gemm(L, x, ids, gates, flags=flags | o.TQ_ROTATE)
    xr = o.hadamard128(x, L.signs)
    sep = o.trellis_expert_gemm(L, xr, ids, gates, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(fused, sep)
    # without signs the rotation is the plain normalised Walsh-Hadamard transform
    L0 = o.TrellisLayer(L.E, L.out, L.in_, L.bits, L.code_off, L.codes, L.scales, None)
    fused0 = o.trellis_expert_gemm(L0, x, ids, flags=flags | o.TQ_ROTATE)
    sep0 = o.trellis_expert_gemm(L0, o.hadamard128(x), ids, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(fused0, sep0)
    ref = oracle_trellis(layer, xr.cpu().numpy().view(np.uint16), ids.cpu().numpy(),
                         gates.cpu().numpy())
    assert rel_l2(fused.cpu().numpy(), ref) <= TOL


def _bf16_bits(v):
    """Round-to-nearest-even bf16 patterns of float values (test input construction)."""
    f = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def test_decode_batch_exact_on_the_token_grid():
    """FORMAT F10: every element within a factor 2^7 of its token's largest magnitude is
    exact on the decode GEMV's 16-bit grid, so only the fp32 summation separates the GPU
    from the exact FP64 result."""
    E, T, topk = 10, 24, 4
    layer = small_layer(413, E, 128, 512)
    rng = rng_for(413, 1)
    # magnitudes 2^-6 .. 2^0 with 8 significant bits: all within 2^7 of the maximum
    mant = rng.integers(128, 256, size=(T, 512)) / 128.0
    expo = rng.integers(-6, 0, size=(T, 512))
    x = _bf16_bits(np.where(rng.random((T, 512)) < 0.5, -1.0, 1.0) * mant * 2.0 ** expo)
    ids = uniform_routes(rng_for(413, 2), T, E, topk)
    y = run(layer, x, ids, flags=1)
    ref = oracle_trellis(layer, x, ids, None)
    assert rel_l2(y, ref) <= 1e-6


def test_decode_batch_outlier_tokens():
    """Tokens whose largest element is 30 and 1000 times their RMS: the decode GEMV rounds
    their small elements to a coarser grid (FORMAT F10); the error stays within the bound
    and grows with the ratio."""
    E, T, topk = 12, 32, 4
    layer = small_layer(414, E, 128, 1024)
    xf = rng_for(414, 1).standard_normal((T, 1024))
    xf[: T // 2, 7] = 30.0
    xf[T // 2:, 700] = -1000.0
    x = _bf16_bits(xf)
    ids = uniform_routes(rng_for(414, 2), T, E, topk)
    y = run(layer, x, ids, flags=1)
    ref = oracle_trellis(layer, x, ids, None)
    e30 = rel_l2(y[: T // 2], ref[: T // 2])
    e1000 = rel_l2(y[T // 2:], ref[T // 2:])
    assert e30 <= 2e-4
    assert e1000 <= TOL


def test_decode_batch_nonfinite_token():
    """A token with an infinite element gives NaN in its slots; the others are unaffected."""
    E, T, topk = 8, 16, 4
    layer = small_layer(415, E, 128, 512)
    x = bf16_from_normal(rng_for(415, 1), (T, 512)).copy()
    x[5, 100] = 0x7F80  # +inf
    ids = uniform_routes(rng_for(415, 2), T, E, topk)
    y = run(layer, x, ids, flags=1)
    assert np.all(np.isnan(y[5]))
    keep = np.arange(T) != 5
    ref = oracle_trellis(layer, x[keep], ids[keep], None)
    assert rel_l2(y[keep], ref) <= TOL


@pytest.mark.timeout(900)
def test_skewed_decode_batch_every_slot():
    # a 128-token decode batch routed by Zipf(1.1) popularity over 384 mixed-width experts:
    # hot experts take dozens of tokens, i.e. several 8-token chunks with waves of their own
    # (some experts with more than 32 pieces, written by the plan's waves); every slot
    # against the oracle
    wl = mixed_layer()
    layer = wl["layer"]
    ids = zipf_routes(rng_for(413, 4), 128, layer["E"], 8)
    counts = np.bincount(ids.reshape(-1), minlength=layer["E"])
    assert counts.max() > 32
    y = run(layer, wl["x"], ids, flags=ops().TQ_GEMV, rotate_signs=layer["signs"])
    ref = oracle_pool.trellis_slots(layer, rotate_host(wl), ids)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL


def test_decode_batch_reduction_prefetch_one_with_many_pieces():
    """The reduction loads one piece ahead of a slot's record when the (group, expert)
    pairs alone could fill the GEMV grid (groups * min(E, N) >= grid). Routes concentrated
    on a few of many experts still give those experts many pieces: the later pieces are
    then loaded after the record, and every one must be added."""
    o = ops()
    # 2,048 experts and 2,048 slots: groups * min(E, N) = 2048, the GEMV grid of a 256-CU
    # GPU at 8 waves per CU, so the reduction prefetches one piece; the slots go to four
    # experts, whose chunks then get several pieces each (up to in / 256 = 8)
    E, T, topk, inp = 2048, 1024, 2, 2048
    layer = small_layer(417, E, 128, inp, widths=np.full(E, 2, np.uint8))
    x = bf16_from_normal(rng_for(417, 1), (T, inp))
    ids = ((np.arange(T * topk, dtype=np.int32) % 3) * 5).reshape(T, topk)  # experts 0, 5, 10
    ids[0, 1] = 7
    y = run(layer, x, ids, flags=o.TQ_GEMV)
    ref = oracle_trellis(layer, x, ids, None)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL


@pytest.mark.parametrize("flags", [1, 2])
def test_token_means_and_magnitudes(flags):
    """Tokens with a large common offset (means 3 and 30: the prefill's byte-sum correction
    removes 255 * sum(x), of order 1e7, from the accumulator), tokens far outside the f16
    range (1e6, 1e30) and far below it (1e-6, 1e-30), a token mixing 1e4 and 1e-4, and a
    token with an infinite element (NaN in its slots only): both modes keep every finite
    token within the bound (each token is put on a power-of-two scale of its own)."""
    E, T, topk, inp = 8, 9, 4, 1024
    layer = small_layer(418, E, 128, inp)
    rng = rng_for(418, 1)
    z = rng.standard_normal((T, inp))
    xf = np.stack([z[0] + 3.0, z[1] + 30.0, z[2] * 1e6, z[3] * 1e30, z[4] * 1e-6,
                   z[5] * 1e-30, np.where(np.arange(inp) % 2 == 0, 1e4, 1e-4) * z[6],
                   z[7], z[8]])
    x = _bf16_bits(xf)
    x[8, 3] = 0x7F80  # +inf
    ids = uniform_routes(rng_for(418, 2), T, E, topk)
    y = run(layer, x, ids, flags=flags)
    assert np.all(np.isnan(y[8]))
    ref = oracle_trellis(layer, x[:8], ids[:8], None)
    for t in range(8):
        pooled, worst = slot_errors(y[t], ref[t])
        assert worst <= TOL, (flags, t, worst)
    assert np.all(np.isfinite(y[:8]))

@pytest.mark.parametrize("flags", [1, 2])
@pytest.mark.parametrize("out_ch", [128, 176, 384])
def test_repacked_layout_gives_the_same_bits(flags, out_ch):
    """trellis_repack copies every unit into the kernels' read order (TQ_LAYOUT_GEMV): the
    results are bit-equal to the store order in both modes, including a last group of fewer
    than 8 strips (out = 176) and several groups (out = 384)."""
    o = ops()
    E, T, topk, inp = 10, 40, 4, 768
    widths = np.array([2, 3, 4, 2, 2, 3, 4, 2, 3, 2], dtype=np.uint8)
    layer = small_layer(419, E, out_ch, inp, widths=widths)
    L = o.TrellisLayer.from_host(layer)
    R = L.repacked()
    assert R.layout == o.TQ_LAYOUT_GEMV and not torch.equal(R.codes, L.codes)
    x = to_dev(bf16_from_normal(rng_for(419, 1), (T, inp)), np.int16)
    ids_h = uniform_routes(rng_for(419, 2), T, E, topk)
    ids_h[2, 1] = -1
    ids = to_dev(ids_h)
    gates = to_dev(softmax_gates(rng_for(419, 3), T, topk))
    for fl in (flags | o.TQ_ROTATE, flags | o.TQ_ROTATE | o.TQ_COMBINE):
        a = o.trellis_expert_gemm(L, x, ids, gates, flags=fl)
        b = o.trellis_expert_gemm(R, x, ids, gates, flags=fl)
        torch.cuda.synchronize()
        assert torch.equal(a, b), fl
    y = o.trellis_expert_gemm(R, x, ids, gates, flags=flags | o.TQ_ROTATE).cpu().numpy()
    xr = oracle.hadamard128_fp32_order(x.cpu().numpy().view(np.uint16), layer["signs"])
    ref = oracle_trellis(layer, xr, ids_h, gates.cpu().numpy())
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL


@pytest.mark.parametrize("flags", [1, 2, 5, 6])
def test_output_side_rotation(flags):
    """A layer with out_signs rotates every 128 outputs of a slot (or of a token with
    TQ_COMBINE) on the output side (FORMAT F17), in both modes, two groups of 128."""
    E, T, topk, inp = 7, 30, 3, 512
    layer = small_layer(420, E, 256, inp)
    layer["out_signs"] = np.where(rng_for(420, 8).integers(0, 2, 256) == 1, 1, -1).astype(np.int8)
    x = bf16_from_normal(rng_for(420, 1), (T, inp))
    ids = uniform_routes(rng_for(420, 2), T, E, topk)
    ids[4, 0] = -1
    gates = softmax_gates(rng_for(420, 3), T, topk)
    y = run(layer, x, ids, gates, flags=flags)
    ref = oracle_trellis(layer, x, ids, gates)
    if flags & 4:
        ref = oracle.combine_slots(ref)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL


@pytest.mark.parametrize("flags", [1, 2])
def test_units128_layout(flags):
    """A layer stored as the exlr8 page's units of 128 inputs (FORMAT F2b,
    TQ_LAYOUT_UNIT128) against the oracle's decode of those units; repacked into the read
    order it gives the same bits."""
    o = ops()
    E, T, topk, inp = 6, 20, 2, 768
    layer = small_layer(421, E, 256, inp)
    layer["layout"] = o.TQ_LAYOUT_UNIT128
    x = bf16_from_normal(rng_for(421, 1), (T, inp))
    ids = uniform_routes(rng_for(421, 2), T, E, topk)
    y = run(layer, x, ids, flags=flags)
    ref = oracle_trellis(layer, x, ids, None)
    pooled, worst = slot_errors(y, ref)
    assert pooled <= TOL and worst <= TOL
    L = o.TrellisLayer.from_host(layer)
    R = L.repacked()
    a = o.trellis_expert_gemm(L, to_dev(x, np.int16), to_dev(ids), flags=flags)
    b = o.trellis_expert_gemm(R, to_dev(x, np.int16), to_dev(ids), flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
