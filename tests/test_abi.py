"""Host-side tests of the C ABI (no GPU): the library loads, exports every function that
include/tq.h declares, and rejects bad arguments with the documented codes before any
HIP call (so these run on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

tq = pytest.importorskip("trellis_quantized_moe_amd")
from trellis_quantized_moe_amd import _lib  # noqa: E402

HEADER = os.path.join(ROOT, "include", "tq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtq.so is not built: run __graft_entry__.build()")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"trellis_expert_gemm", "mxfp4_expert_gemm", "hadamard128"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_version(lib):
    assert lib.tq_version() == 100


def _layer(E=4, out=128, inp=5120, fake=0x1000, signs=None, codes_bytes=1 << 30):
    return _lib.TrellisLayerC(E, out, inp, 0, fake, fake, fake, fake, signs, codes_bytes, None)


def _call_trellis(lib, layer, T=2, topk=2, x=0x1000, ids=0x1000, y=0x1000, flags=0,
                  ws=0x10000, ws_bytes=1 << 30):
    return lib.trellis_expert_gemm(ctypes.byref(layer), x, T, ids, None, topk, y, flags, ws,
                                   ws_bytes, None)


def test_trellis_argument_errors(lib):
    assert lib.trellis_expert_gemm(None, 0x1000, 1, 0x1000, None, 1, 0x1000, 0, 0x1000, 1 << 30,
                                   None) == _lib.TQ_EINVAL
    for bad in (_layer(E=0), _layer(out=24), _layer(inp=200), _layer(E=70000)):
        assert _call_trellis(lib, bad) == _lib.TQ_EINVAL
    lay = _layer()
    lay.layout = 3
    assert _call_trellis(lib, lay) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(codes_bytes=0)) == _lib.TQ_EINVAL
    assert b"codes_bytes" in lib.tq_last_error()
    lay = _layer(out=144)
    lay.out_signs = 0x1000
    assert _call_trellis(lib, lay) == _lib.TQ_EINVAL  # output rotation needs out % 128 == 0
    lay = _layer()
    lay.layout = _lib.TQ_LAYOUT_UNIT128
    lay.in_ = 5120 + 64 * 3  # not a multiple of 128 (but of 64)
    assert _call_trellis(lib, lay) == _lib.TQ_EINVAL
    lay = _layer()
    lay.codes = 0x1008
    assert _call_trellis(lib, lay) == _lib.TQ_EALIGN
    assert _call_trellis(lib, _layer(), topk=0) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), topk=65) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), T=-1) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), T=1 << 30, topk=4) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), flags=3) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), flags=32) == _lib.TQ_EINVAL
    # the FP8 variant is a prefill-mode contraction: not with the decode batch
    assert _call_trellis(lib, _layer(), flags=_lib.TQ_FP8 | 1) == _lib.TQ_EINVAL
    # codebooks: only 0..2; mul1 and pmcgx need TQ_FP8 and a store or read-order layout
    lay = _layer()
    lay.codebook = 3
    assert _call_trellis(lib, lay) == _lib.TQ_EINVAL
    lay.codebook = _lib.TQ_CODEBOOK_PMCGX
    assert _call_trellis(lib, lay, flags=_lib.TQ_GEMM) == _lib.TQ_EINVAL
    assert b"TQ_FP8" in lib.tq_last_error()
    lay.layout = 2
    assert _call_trellis(lib, lay, flags=_lib.TQ_FP8) == _lib.TQ_EINVAL
    # TQ_ROTATE reads 16 signs per tile column: the signs must be 16-byte aligned
    assert _call_trellis(lib, _layer(signs=0x1008), flags=_lib.TQ_ROTATE) == _lib.TQ_EALIGN
    assert _call_trellis(lib, _layer(), x=0x1002) == _lib.TQ_EALIGN
    assert _call_trellis(lib, _layer(), y=0) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), ids=0) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(), ws=0) == _lib.TQ_EWORKSPACE
    assert _call_trellis(lib, _layer(), ws=0x10010) == _lib.TQ_EALIGN
    assert _call_trellis(lib, _layer(), ws_bytes=16) == _lib.TQ_EWORKSPACE
    assert b"workspace" in lib.tq_last_error()
    # layers are limited to E <= 4096 (both modes)
    assert _call_trellis(lib, _layer(E=5000), T=100000, topk=8, flags=_lib.TQ_GEMM) == _lib.TQ_EINVAL
    assert _call_trellis(lib, _layer(E=5000), T=4, topk=8, flags=_lib.TQ_GEMV) == _lib.TQ_EINVAL


def test_empty_batch_is_a_no_op(lib):
    # T == 0 succeeds without touching the device (no workspace needed either)
    assert _call_trellis(lib, _layer(), T=0, x=0, ids=0, y=0, ws=0, ws_bytes=0) == _lib.TQ_OK
    assert lib.tq_last_error() == b""
    m = _lib.Mxfp4LayerC(4, 128, 5120, 0, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0, 0, 0, None, 8, 0, 0, 0, 0, None) == _lib.TQ_OK
    assert lib.hadamard128(0, 0, 0, 128, None, None) == _lib.TQ_OK


def test_mxfp4_argument_errors(lib):
    m = _lib.Mxfp4LayerC(4, 128, 5120 + 256, 0, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0x1000, 1, 0x1000, None, 1, 0x1000, 0, 0x1000,
                                 1 << 30, None) == _lib.TQ_EINVAL
    m = _lib.Mxfp4LayerC(4, 128, 5120, 0, 0x1001)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0x1000, 1, 0x1000, None, 1, 0x1000, 0, 0x1000,
                                 1 << 30, None) == _lib.TQ_EALIGN
    # the input rotation is a trellis-layer option
    m = _lib.Mxfp4LayerC(4, 128, 5120, 0, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0x1000, 1, 0x1000, None, 1, 0x1000,
                                 _lib.TQ_ROTATE, 0x1000, 1 << 30, None) == _lib.TQ_EINVAL


def test_fp8b32_argument_errors(lib):
    ok = _lib.Mxfp4LayerC(1, 1536, 5120, 0, 0x1000)
    assert lib.fp8b32_expert_gemm(ctypes.byref(ok), 0, 0, 0, None, 1, 0, 0, 0, 0, None) == _lib.TQ_OK
    for bad in (_lib.Mxfp4LayerC(0, 128, 5120, 0, 0x1000), _lib.Mxfp4LayerC(1, 48, 5120, 0, 0x1000),
                _lib.Mxfp4LayerC(1, 128, 5120 + 128, 0, 0x1000), _lib.Mxfp4LayerC(1, 128, 5120, 2, 0x1000)):
        assert lib.fp8b32_expert_gemm(ctypes.byref(bad), 0x1000, 1, 0x1000, None, 1, 0x1000, 0,
                                      0x1000, 1 << 30, None) == _lib.TQ_EINVAL
    mis = _lib.Mxfp4LayerC(1, 128, 5120, 0, 0x1008)
    assert lib.fp8b32_expert_gemm(ctypes.byref(mis), 0x1000, 1, 0x1000, None, 1, 0x1000, 0, 0x1000,
                                  1 << 30, None) == _lib.TQ_EALIGN
    assert lib.fp8b32_expert_gemm(ctypes.byref(ok), 0x1000, 1, 0x1000, None, 1, 0x1000,
                                  _lib.TQ_ROTATE, 0x1000, 1 << 30, None) == _lib.TQ_EINVAL
    assert lib.fp8b32_decode(0x1000, 48, 64, 0x1000, None) == _lib.TQ_EINVAL
    assert lib.fp8b32_decode(0x1000, 32, 48, 0x1000, None) == _lib.TQ_EINVAL
    assert lib.fp8b32_decode(0x1008, 32, 64, 0x1000, None) == _lib.TQ_EALIGN


def test_repack_argument_errors(lib):
    for fn in (lib.mxfp4_repack, lib.fp8b32_repack):
        store = _lib.Mxfp4LayerC(2, 128, 5120, _lib.TQ_LAYOUT_STORE, 0x100000)
        packed = _lib.Mxfp4LayerC(2, 128, 5120, _lib.TQ_LAYOUT_GEMV, 0x100000)
        assert fn(None, 0x1000, None) == _lib.TQ_EINVAL
        assert fn(ctypes.byref(packed), 0x10000000, None) == _lib.TQ_EINVAL   # already repacked
        assert fn(ctypes.byref(store), None, None) == _lib.TQ_EINVAL
        assert fn(ctypes.byref(store), 0x10000008, None) == _lib.TQ_EALIGN
        assert fn(ctypes.byref(store), 0x100010, None) == _lib.TQ_EINVAL      # overlaps the units
    bad = _lib.Mxfp4LayerC(4, 128, 5120, 2, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(bad), 0x1000, 1, 0x1000, None, 1, 0x1000, 0, 0x1000,
                                 1 << 30, None) == _lib.TQ_EINVAL


def test_decode_batch_wave_bound(lib):
    # 4096 experts of 1024 outputs (8 groups): 8 * (4096 + ceil(1 / 16)) (group, chunk) pairs
    # exceed the 32768 launched waves of a decode batch: forced decode is rejected before
    # any device work, and the automatic choice takes the prefill path (its workspace)
    m = _lib.Mxfp4LayerC(4096, 1024, 512, 0, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0x1000, 1, 0x1000, None, 1, 0x1000,
                                 _lib.TQ_GEMV, 0x1000, 1 << 30, None) == _lib.TQ_EINVAL
    assert b"32768" in lib.tq_last_error()
    auto = lib.tq_workspace_bytes(1, 1, 4096, 1024, 512, _lib.TQ_AUTO)
    gemm = lib.tq_workspace_bytes(1, 1, 4096, 1024, 512, _lib.TQ_GEMM)
    assert auto == gemm
    # one group fewer fits: 7 * 4097 <= 32768
    m = _lib.Mxfp4LayerC(4096, 896, 512, 0, 0x1000)
    assert lib.mxfp4_expert_gemm(ctypes.byref(m), 0x1000, 1, 0x1000, None, 1, 0x1000,
                                 _lib.TQ_GEMV, 0x1000, 8, None) == _lib.TQ_EWORKSPACE


def test_internal_helpers_are_not_exported(lib):
    for name in ("common_checks", "check_trellis_layer", "check_mxfp4_layer", "run_route",
                 "ffn_ws", "mx_unit_bytes"):
        assert not hasattr(lib, name), name


def test_hadamard_decode_route_argument_errors(lib):
    assert lib.hadamard128(0x1000, 0x1000, 1, 100, None, None) == _lib.TQ_EINVAL
    assert lib.hadamard128(0x1000, 0x1000, -1, 128, None, None) == _lib.TQ_EINVAL
    assert lib.hadamard128(0x1001, 0x1000, 1, 128, None, None) == _lib.TQ_EALIGN
    assert lib.hadamard128(0x1000, 0x1000, 1, 128, 0x1004, None) == _lib.TQ_EALIGN
    assert lib.trellis_decode(0x1000, 5, 16, 64, 0x1000, 0, None) == _lib.TQ_EINVAL
    assert lib.trellis_decode(0x1000, 2, 17, 64, 0x1000, 0, None) == _lib.TQ_EINVAL
    assert lib.trellis_decode(0x1000, 2, 16, 48, 0x1000, 0, None) == _lib.TQ_EINVAL
    assert lib.trellis_decode(0x1000, 2, 16, 64, 0x1000, 5, None) == _lib.TQ_EINVAL
    assert lib.trellis_decode(0x1004, 2, 16, 64, 0x1000, 0, None) == _lib.TQ_EALIGN
    assert lib.mxfp4_decode(0x1000, 16, 48, 0x1000, None) == _lib.TQ_EINVAL
    m = _lib.Mxfp4LayerC(4, 128, 5120, 0, 0x1000)
    assert lib.mxfp4_to_nvfp4(None, 0x1000, 0x1000, 0x1000, 0x1000, None) == _lib.TQ_EINVAL
    for bad in (_lib.Mxfp4LayerC(0, 128, 5120, 0, 0x1000), _lib.Mxfp4LayerC(4, 24, 5120, 0, 0x1000),
                _lib.Mxfp4LayerC(4, 128, 1000, 0, 0x1000), _lib.Mxfp4LayerC(4, 128, 5120, 1, 0x1000)):
        assert lib.mxfp4_to_nvfp4(ctypes.byref(bad), 0x1000, 0x1000, 0x1000, 0x1000, None) == _lib.TQ_EINVAL
    assert lib.mxfp4_to_nvfp4(ctypes.byref(m), None, 0x1000, 0x1000, 0x1000, None) == _lib.TQ_EINVAL
    assert lib.mxfp4_to_nvfp4(ctypes.byref(m), 0x1008, 0x1000, 0x1000, 0x1000, None) == _lib.TQ_EALIGN
    assert lib.mxfp4_to_nvfp4(ctypes.byref(m), 0x1000, 0x1000, 0x1002, 0x1000, None) == _lib.TQ_EALIGN
    assert lib.route_bucket(0x1000, 4, 2, 0, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 20, None) == _lib.TQ_EINVAL
    assert lib.route_bucket(0x1000, 4, 2, 5000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 20, None) == _lib.TQ_EINVAL
    assert lib.route_bucket(0x1000, 4, 2, 8, 0x1000, 0x1000, 0x1000, 0x1000, 8, None) == _lib.TQ_EWORKSPACE
    v = ctypes.c_uint32(0)
    assert lib.tq_device_status(None, None, ctypes.byref(v)) == _lib.TQ_EINVAL


def test_workspace_sizes(lib):
    # decode batch: counters + slice partials; prefill: route buffers and items
    gemv = lib.tq_workspace_bytes(128, 8, 384, 128, 5120, _lib.TQ_AUTO)
    gemm = lib.tq_workspace_bytes(8192, 8, 384, 128, 5120, _lib.TQ_AUTO)
    assert gemv >= 256 + 384 * 4 + 4 * 1024 * 128 * 4
    assert gemm >= 256 + 8192 * 8 * 4 * 2 + (8192 * 8 // 128 + 384) * 16
    comb = lib.tq_workspace_bytes(8192, 8, 384, 128, 5120, _lib.TQ_COMBINE)
    assert comb >= gemm + 8192 * 8 * 128 * 4
    assert lib.tq_workspace_bytes(-1, 8, 384, 128, 5120, 0) == 0
