"""PyTorch-facing wrappers of the C ABI: device tensors in, device tensors out.

PyTorch supplies device memory and the current stream; each call passes raw pointers to
libtq.so, which enqueues the gfx950 kernels on that stream. No computation happens here.
"""

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import (TQ_AUTO, TQ_COMBINE, TQ_GEMM, TQ_GEMV, TQ_LAYOUT_GEMV,  # noqa: F401
                   TQ_LAYOUT_STORE, TQ_LAYOUT_UNIT128, TQ_ROTATE, TQ_FP8, TQ_CODEBOOK_T16,
                   TQ_CODEBOOK_MUL1, TQ_CODEBOOK_PMCGX, check)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


@dataclass
class TrellisLayer:
    """A trellis expert layer in device memory (see tq_trellis_layer in include/tq.h)."""
    E: int
    out: int
    in_: int
    bits: torch.Tensor       # uint8 [E]
    code_off: torch.Tensor   # int64 [E], byte offsets
    codes: torch.Tensor      # int32 [words] (uint32 bit patterns)
    scales: torch.Tensor     # int16 [E, out] (fp16 bit patterns)
    signs: torch.Tensor = None  # int8 [in] rotation signs (TQ_ROTATE), or None
    layout: int = TQ_LAYOUT_STORE
    out_signs: torch.Tensor = None  # int8 [out] output-side rotation signs, or None
    codebook: int = 0               # TQ_CODEBOOK_T16, _MUL1 or _PMCGX

    @classmethod
    def from_host(cls, layer, device="cuda"):
        signs = layer.get("signs")
        out_signs = layer.get("out_signs")
        return cls(
            E=int(layer["E"]), out=int(layer["out"]), in_=int(layer["in"]),
            bits=torch.from_numpy(np.ascontiguousarray(layer["bits"], dtype=np.uint8)).to(device),
            code_off=torch.from_numpy(np.ascontiguousarray(layer["code_off"], dtype=np.int64)).to(device),
            codes=torch.from_numpy(np.ascontiguousarray(layer["codes"]).view(np.int32)).to(device),
            scales=torch.from_numpy(np.ascontiguousarray(layer["scales"]).view(np.int16)).to(device),
            signs=None if signs is None else
            torch.from_numpy(np.ascontiguousarray(signs, dtype=np.int8)).to(device),
            layout=int(layer.get("layout", TQ_LAYOUT_STORE)),
            out_signs=None if out_signs is None else
            torch.from_numpy(np.ascontiguousarray(out_signs, dtype=np.int8)).to(device),
            codebook=int(layer.get("codebook", 0)),
        )

    def with_codes(self, codes):
        """The same layer reading its units from another copy of the code buffer."""
        return TrellisLayer(self.E, self.out, self.in_, self.bits, self.code_off, codes,
                            self.scales, self.signs, self.layout, self.out_signs, self.codebook)

    def repacked(self):
        """The same layer with its units copied into TQ_LAYOUT_GEMV (see trellis_repack in
        include/tq.h)."""
        _require_cuda(self.codes)
        dst = torch.zeros_like(self.codes)
        c = self.c_struct()
        check(_lib.load().trellis_repack(ctypes.byref(c), _ptr(dst), _stream(self.codes.device)))
        return TrellisLayer(self.E, self.out, self.in_, self.bits, self.code_off, dst,
                            self.scales, self.signs, TQ_LAYOUT_GEMV, self.out_signs,
                            self.codebook)

    def c_struct(self):
        return _lib.TrellisLayerC(self.E, self.out, self.in_, self.layout, self.bits.data_ptr(),
                                  self.code_off.data_ptr(), self.codes.data_ptr(),
                                  self.scales.data_ptr(),
                                  None if self.signs is None else self.signs.data_ptr(),
                                  self.codes.numel() * self.codes.element_size(),
                                  None if self.out_signs is None else self.out_signs.data_ptr(),
                                  self.codebook)


@dataclass
class Mxfp4Layer:
    """An MXFP4 expert layer in device memory (see tq_mxfp4_layer in include/tq.h)."""
    E: int
    out: int
    in_: int
    units: torch.Tensor      # uint8 [E * unit_bytes]
    layout: int = TQ_LAYOUT_STORE

    @classmethod
    def from_host(cls, layer, device="cuda"):
        return cls(E=int(layer["E"]), out=int(layer["out"]), in_=int(layer["in"]),
                   units=torch.from_numpy(np.ascontiguousarray(layer["units"], dtype=np.uint8)).to(device))

    def with_units(self, units):
        return Mxfp4Layer(self.E, self.out, self.in_, units, self.layout)

    def c_struct(self):
        return _lib.Mxfp4LayerC(self.E, self.out, self.in_, self.layout, self.units.data_ptr())

    def repacked(self):
        """The same layer with its units copied into TQ_LAYOUT_GEMV (see mxfp4_repack in
        include/tq.h)."""
        _require_cuda(self.units)
        dst = torch.empty_like(self.units)
        c = self.c_struct()
        check(_lib.load().mxfp4_repack(ctypes.byref(c), _ptr(dst), _stream(self.units.device)))
        return Mxfp4Layer(self.E, self.out, self.in_, dst, TQ_LAYOUT_GEMV)


@dataclass
class Fp8b32Layer:
    """An fp8b32 expert layer in device memory (see tq_fp8b32_layer in include/tq.h)."""
    E: int
    out: int
    in_: int
    units: torch.Tensor      # uint8 [E * unit_bytes]
    layout: int = TQ_LAYOUT_STORE

    @classmethod
    def from_host(cls, layer, device="cuda"):
        return cls(E=int(layer["E"]), out=int(layer["out"]), in_=int(layer["in"]),
                   units=torch.from_numpy(np.ascontiguousarray(layer["units"], dtype=np.uint8)).to(device))

    def with_units(self, units):
        return Fp8b32Layer(self.E, self.out, self.in_, units, self.layout)

    def c_struct(self):
        return _lib.Mxfp4LayerC(self.E, self.out, self.in_, self.layout, self.units.data_ptr())

    def repacked(self):
        """The same layer with its units copied into TQ_LAYOUT_GEMV (see fp8b32_repack in
        include/tq.h)."""
        _require_cuda(self.units)
        dst = torch.empty_like(self.units)
        c = self.c_struct()
        check(_lib.load().fp8b32_repack(ctypes.byref(c), _ptr(dst), _stream(self.units.device)))
        return Fp8b32Layer(self.E, self.out, self.in_, dst, TQ_LAYOUT_GEMV)


def workspace_bytes(T, topk, E, out, in_, flags=TQ_AUTO):
    return int(_lib.load().tq_workspace_bytes(T, topk, E, out, in_, flags))


def workspace(T, topk, E, out, in_, flags=TQ_AUTO, device="cuda"):
    """A zero-filled workspace (the library requires zeros before the first use)."""
    n = max(256, workspace_bytes(T, topk, E, out, in_, flags))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def hadamard128(x, signs=None, out=None):
    """bf16 [rows, n] -> bf16 [rows, n], 128-wide rotation (x may be bf16/int16/uint16)."""
    _require_cuda(x, signs, out)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, n] tensor")
    y = torch.empty_like(x) if out is None else out
    check(_lib.load().hadamard128(_ptr(x), _ptr(y), x.shape[0], x.shape[1], _ptr(signs),
                                  _stream(x.device)))
    return y


def mxfp8_quantize(x):
    """(codes uint8 [rows, n], scales uint8 [rows, n / 32]): the MXFP8 form of bf16 rows (see
    mxfp8_quantize in include/tq.h)."""
    _require_cuda(x)
    rows, n = x.shape
    codes = torch.empty((rows, n), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, n // 32), dtype=torch.uint8, device=x.device)
    check(_lib.load().mxfp8_quantize(_ptr(x), rows, n, _ptr(codes), _ptr(scales),
                                     _stream(x.device)))
    return codes, scales


def _gemm(fn, layer_c, E, out_ch, in_, x, topk_ids, topk_w, flags, out, ws, mxfp4):
    _require_cuda(x, topk_ids, topk_w, out, ws)
    T, topk = topk_ids.shape
    if out is None:
        shape = (T, out_ch) if flags & TQ_COMBINE else (T, topk, out_ch)
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(T, topk, E, out_ch, in_, flags, device=x.device)
    check(fn(ctypes.byref(layer_c), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), topk, _ptr(out),
             flags, _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def trellis_expert_gemm(layer, x, topk_ids, topk_w=None, flags=TQ_AUTO, out=None, ws=None):
    """fp32 per-slot outputs [T, topk, out] (or [T, out] with TQ_COMBINE)."""
    return _gemm(_lib.load().trellis_expert_gemm, layer.c_struct(), layer.E, layer.out,
                 layer.in_, x, topk_ids, topk_w, flags, out, ws, False)


def trellis_expert_gemm_noalloc(layer, x, topk_ids, topk_w=None, flags=TQ_AUTO, out=None):
    """trellis_expert_gemm with the library's static device scratch as its workspace (see
    trellis_expert_gemm_noalloc in include/tq.h). `out` must be given for the call itself
    to allocate nothing."""
    _require_cuda(x, topk_ids, topk_w, out)
    T, topk = topk_ids.shape
    if out is None:
        shape = (T, layer.out) if flags & TQ_COMBINE else (T, topk, layer.out)
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    layer_c = layer.c_struct()
    check(_lib.load().trellis_expert_gemm_noalloc(ctypes.byref(layer_c), _ptr(x), T,
                                                  _ptr(topk_ids), _ptr(topk_w), topk, _ptr(out),
                                                  flags, _stream(x.device)))
    return out


def mxfp4_expert_gemm(layer, x, topk_ids, topk_w=None, flags=TQ_AUTO, out=None, ws=None):
    return _gemm(_lib.load().mxfp4_expert_gemm, layer.c_struct(), layer.E, layer.out,
                 layer.in_, x, topk_ids, topk_w, flags, out, ws, True)


def fp8b32_expert_gemm(layer, x, topk_ids, topk_w=None, flags=TQ_AUTO, out=None, ws=None):
    return _gemm(_lib.load().fp8b32_expert_gemm, layer.c_struct(), layer.E, layer.out,
                 layer.in_, x, topk_ids, topk_w, flags, out, ws, True)


def route_bucket(topk_ids, E, ws=None):
    """(counts [E], offsets [E+1], pairs [T*topk]) as int32 device tensors."""
    _require_cuda(topk_ids, ws)
    T, topk = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pairs = torch.full((max(1, T * topk),), -1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(T, topk, E, 16, 256, TQ_GEMM, device=dev)
    check(_lib.load().route_bucket(_ptr(topk_ids), T, topk, E, _ptr(counts), _ptr(offsets),
                                   _ptr(pairs), _ptr(ws), ws.numel(), _stream(dev)))
    return counts, offsets, pairs[:T * topk]


def trellis_decode(codes, K, out_ch, in_, path=0):
    """int16 q [out, in] of one unit, via the GEMV (path 0) or prefill (path 1) decoder; path
    2 gives the E4M3 codes of the FP8 prefill's decoder."""
    _require_cuda(codes)
    q = torch.empty((out_ch, in_), dtype=torch.int16, device=codes.device)
    check(_lib.load().trellis_decode(_ptr(codes), K, out_ch, in_, _ptr(q), path,
                                     _stream(codes.device)))
    return q


def mxfp4_decode(unit, out_ch, in_):
    """bf16 bit patterns (int16) [out, in] of one MXFP4 unit."""
    _require_cuda(unit)
    w = torch.empty((out_ch, in_), dtype=torch.int16, device=unit.device)
    check(_lib.load().mxfp4_decode(_ptr(unit), out_ch, in_, _ptr(w), _stream(unit.device)))
    return w


def fp8b32_decode(unit, out_ch, in_):
    """bf16 bit patterns (int16) [out, in] of one fp8b32 unit."""
    _require_cuda(unit)
    w = torch.empty((out_ch, in_), dtype=torch.int16, device=unit.device)
    check(_lib.load().fp8b32_decode(_ptr(unit), out_ch, in_, _ptr(w), _stream(unit.device)))
    return w


def ffn_workspace(T, topk, E, H, I, flags=TQ_AUTO, device="cuda"):
    n = max(256, int(_lib.load().tq_ffn_workspace_bytes(T, topk, E, H, I, flags)))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def trellis_expert_ffn(gate_up, down, x, topk_ids, topk_w=None, flags=TQ_AUTO, out=None,
                       ws=None):
    """fp32 [T, H]: the routed expert FFN over a fused trellis gate/up layer (out = 2I) and a
    trellis down layer (see trellis_expert_ffn in include/tq.h)."""
    _require_cuda(x, topk_ids, topk_w, out, ws)
    T, topk = topk_ids.shape
    if out is None:
        out = torch.empty((T, gate_up.in_), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = ffn_workspace(T, topk, gate_up.E, gate_up.in_, gate_up.out // 2, flags,
                           device=x.device)
    gu, d = gate_up.c_struct(), down.c_struct()
    check(_lib.load().trellis_expert_ffn(ctypes.byref(gu), ctypes.byref(d), _ptr(x), T,
                                         _ptr(topk_ids), _ptr(topk_w), topk, _ptr(out), flags,
                                         _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def mxfp4_to_nvfp4(layer, codes=None, scales=None, scale2=None, status=None):
    """NVFP4 form of an MXFP4 layer: (codes uint8 [E, out*in/2], scales uint8 [E, out, in/16],
    scale2 fp32 [E], status uint8 [E]) (see mxfp4_to_nvfp4 in include/tq.h)."""
    _require_cuda(layer.units, codes, scales, scale2, status)
    dev = layer.units.device
    E, out_ch, in_ = layer.E, layer.out, layer.in_
    if codes is None:
        codes = torch.empty((E, out_ch * in_ // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((E, out_ch, in_ // 16), dtype=torch.uint8, device=dev)
    if scale2 is None:
        scale2 = torch.empty(E, dtype=torch.float32, device=dev)
    if status is None:
        status = torch.empty(E, dtype=torch.uint8, device=dev)
    c = layer.c_struct()
    check(_lib.load().mxfp4_to_nvfp4(ctypes.byref(c), _ptr(codes), _ptr(scales), _ptr(scale2),
                                     _ptr(status), _stream(dev)))
    return codes, scales, scale2, status


def device_status(ws):
    """Synchronise, read and clear the workspace status bits."""
    v = ctypes.c_uint32(0)
    check(_lib.load().tq_device_status(_ptr(ws), _stream(ws.device), ctypes.byref(v)))
    return v.value


def version():
    return int(_lib.load().tq_version())


def time_kernel(start, stop):
    """Measurement hook: the next expert GEMM or FFN call on this thread sets the
    torch.cuda.Event pair (start, stop) to its main kernel's own start and end
    (tq_time_kernel)."""
    if start is None:
        check(_lib.load().tq_time_kernel(None, None))
        return
    check(_lib.load().tq_time_kernel(ctypes.c_void_p(start.cuda_event),
                                      ctypes.c_void_p(stop.cuda_event)))
