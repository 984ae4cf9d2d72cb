"""ctypes loader for libtq.so (the C ABI declared in include/tq.h).

Argument marshalling only: every computation happens in the gfx950 kernels behind the
ABI. Loading fails loudly when the library has not been built.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK = 0
TQ_EINVAL = -1
TQ_EUNSUPPORTED = -2
TQ_EALIGN = -3
TQ_EWORKSPACE = -4
TQ_EHIP = -5

TQ_LAYOUT_STORE = 0
TQ_LAYOUT_GEMV = 1
TQ_LAYOUT_UNIT128 = 2

TQ_AUTO = 0
TQ_GEMV = 1
TQ_GEMM = 2
TQ_COMBINE = 4
TQ_ROTATE = 8
TQ_FP8 = 16
TQ_CODEBOOK_T16, TQ_CODEBOOK_MUL1, TQ_CODEBOOK_PMCGX = 0, 1, 2

TQ_NOALLOC_SCRATCH_BYTES = 32 << 20

TQ_STATUS_BAD_EXPERT = 1
TQ_STATUS_BAD_UNIT = 2


class TrellisLayerC(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32),
        ("out", ctypes.c_int32),
        ("in_", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("bits", ctypes.c_void_p),
        ("code_off", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("signs", ctypes.c_void_p),
        ("codes_bytes", ctypes.c_int64),
        ("out_signs", ctypes.c_void_p),
        ("codebook", ctypes.c_int32),
    ]


class Mxfp4LayerC(ctypes.Structure):
    # also the layout of tq_fp8b32_layer (same fields)
    _fields_ = [
        ("E", ctypes.c_int32),
        ("out", ctypes.c_int32),
        ("in_", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("units", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t

SIGNATURES = {
    "trellis_expert_gemm": (ctypes.c_int, [ctypes.POINTER(TrellisLayerC), _P, _I64, _P, _P, _I32,
                                           _P, _U32, _P, _SZ, _P]),
    "mxfp4_expert_gemm": (ctypes.c_int, [ctypes.POINTER(Mxfp4LayerC), _P, _I64, _P, _P, _I32,
                                         _P, _U32, _P, _SZ, _P]),
    "hadamard128": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "mxfp8_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "route_bucket": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "trellis_decode": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _P]),
    "mxfp4_decode": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "fp8b32_expert_gemm": (ctypes.c_int, [ctypes.POINTER(Mxfp4LayerC), _P, _I64, _P, _P, _I32,
                                          _P, _U32, _P, _SZ, _P]),
    "fp8b32_decode": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "trellis_repack": (ctypes.c_int, [ctypes.POINTER(TrellisLayerC), _P, _P]),
    "mxfp4_repack": (ctypes.c_int, [ctypes.POINTER(Mxfp4LayerC), _P, _P]),
    "fp8b32_repack": (ctypes.c_int, [ctypes.POINTER(Mxfp4LayerC), _P, _P]),
    "mxfp4_to_nvfp4": (ctypes.c_int, [ctypes.POINTER(Mxfp4LayerC), _P, _P, _P, _P, _P]),
    "trellis_expert_ffn": (ctypes.c_int, [ctypes.POINTER(TrellisLayerC), ctypes.POINTER(TrellisLayerC),
                                          _P, _I64, _P, _P, _I32, _P, _U32, _P, _SZ, _P]),
    "trellis_expert_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(TrellisLayerC), _P, _I64, _P,
                                                   _P, _I32, _P, _U32, _P]),
    "tq_ffn_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _U32]),
    "tq_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _U32]),
    "tq_last_error": (ctypes.c_char_p, []),
    "tq_device_status": (ctypes.c_int, [_P, _P, ctypes.POINTER(_U32)]),
    "tq_version": (ctypes.c_int, []),
    "tq_time_kernel": (ctypes.c_int, [_P, _P]),
}

_lib = None


def load():
    """The loaded library (cached). Raises if libtq.so is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libtq.so is not built (%s); run trellis_quantized_moe_amd.build.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class TQError(RuntimeError):
    def __init__(self, code, message):
        super().__init__("tq error %d: %s" % (code, message))
        self.code = code


def check(rc):
    if rc != TQ_OK:
        raise TQError(rc, load().tq_last_error().decode())
    return rc
