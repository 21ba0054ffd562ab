"""Python binding of libmoe.so (include/moe.h): argument marshalling only.

Every step of the routed-expert FFN runs in the library's HIP kernels; this
module passes device pointers (torch tensors) and the current HIP stream.
It raises if the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names another build of the same library (the host-only
# sanitizer flavour of the host tests); it must exist like the default one
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_AFFINE, MOE_SYMMETRIC, MOE_DENSE = 0, 1, 2
MOE_BF16, MOE_FP16 = 0, 1


class MoeError(RuntimeError):
    pass


class QFormatC(C.Structure):
    _fields_ = [("bits", C.c_int32), ("group", C.c_int32), ("mode", C.c_int32),
                ("scale_dtype", C.c_int32)]


class LayerDescC(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("act_dtype", C.c_int32),
                ("router", QFormatC), ("gate_row", QFormatC), ("routed", QFormatC),
                ("shared", QFormatC)]


class QTensorC(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p)]


class LayerSrcC(C.Structure):
    _fields_ = [(n, QTensorC) for n in
                ("router", "gate_row", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")]


class MatOffC(C.Structure):
    _fields_ = [("codes", C.c_uint64), ("scales", C.c_uint64)]


class LayerC(C.Structure):
    _fields_ = [("d", LayerDescC), ("dev", C.c_void_p), ("bytes", C.c_uint64),
                ("router_off", C.c_uint64), ("router_scale_off", C.c_uint64),
                ("gate_row_off", C.c_uint64), ("gate_row_scale_off", C.c_uint64),
                ("experts_off", C.c_uint64), ("expert_stride", C.c_uint64),
                ("gu", MatOffC), ("dn", MatOffC), ("shared_off", C.c_uint64),
                ("sh_gu", MatOffC), ("sh_dn", MatOffC), ("flags", C.c_uint32)]


class TapsC(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("gu", C.c_void_p), ("h", C.c_void_p), ("e", C.c_void_p),
                ("kernel_events", C.c_void_p * 8), ("route_wait_limit", C.c_int32)]


EXPORTS = ["moe_pack_size", "moe_pack_layer_host", "moe_layer_bind", "moe_pack_layer",
           "moe_workspace_size", "moe_route", "moe_experts_decode", "moe_experts_grouped",
           "moe_forward_windows", "moe_forward_windows_noalloc", "moe_route_failures",
           "moe_forward_exact", "moe_status_string", "moe_last_error", "moe_version"]

MOE_WS_DECODE, MOE_WS_GROUPED, MOE_WS_EXACT = 0, 1, 2

_lib = None


def lib() -> C.CDLL:
    """Loads libmoe.so (built in-tree by build()); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is missing: build it first "
                       "(python -m quantized_routed_expert_fp32_amd.csrc.build)")
    L = C.CDLL(LIB_PATH)
    vp, i32, u64 = C.c_void_p, C.c_int32, C.c_uint64
    L.moe_pack_size.argtypes = [C.POINTER(LayerDescC), C.POINTER(u64)]
    L.moe_pack_layer_host.argtypes = [C.POINTER(LayerDescC), C.POINTER(LayerSrcC), vp, u64,
                                      C.POINTER(LayerC)]
    L.moe_layer_bind.argtypes = [C.POINTER(LayerC), vp]
    L.moe_pack_layer.argtypes = [C.POINTER(LayerDescC), C.POINTER(LayerSrcC), vp, u64, vp,
                                 C.POINTER(LayerC)]
    L.moe_workspace_size.argtypes = [C.POINTER(LayerDescC), i32, i32, C.POINTER(u64)]
    L.moe_route.argtypes = [C.POINTER(LayerC), vp, i32, vp, vp, vp, vp, vp, u64, C.POINTER(TapsC),
                            vp]
    L.moe_experts_decode.argtypes = [C.POINTER(LayerC), vp, i32, vp, vp, vp, vp, vp, u64,
                                     C.POINTER(TapsC), vp]
    L.moe_experts_grouped.argtypes = L.moe_experts_decode.argtypes
    L.moe_forward_windows.argtypes = [C.POINTER(LayerC), vp, i32, vp, vp, vp, vp, vp, vp, u64, vp]
    L.moe_route_failures.argtypes = [vp, u64, i32, C.POINTER(C.c_uint32), vp]
    L.moe_forward_windows_noalloc.argtypes = [C.POINTER(LayerC), vp, i32, vp, vp, vp, vp, vp, vp]
    L.moe_forward_exact.argtypes = [C.POINTER(LayerC), vp, i32, vp, vp, vp, vp, vp, vp, u64,
                                    C.POINTER(TapsC), vp]
    for f in ("moe_pack_size", "moe_pack_layer_host", "moe_layer_bind", "moe_pack_layer",
              "moe_workspace_size", "moe_route", "moe_experts_decode", "moe_experts_grouped",
              "moe_forward_windows", "moe_forward_windows_noalloc", "moe_route_failures",
              "moe_forward_exact"):
        getattr(L, f).restype = C.c_int
    L.moe_status_string.argtypes = [C.c_int]
    L.moe_status_string.restype = C.c_char_p
    L.moe_last_error.restype = C.c_char_p
    L.moe_version.restype = C.c_char_p
    _lib = L
    return L


def _check(st: int, what: str):
    if st != 0:
        L = lib()
        raise MoeError(f"{what}: {L.moe_status_string(st).decode()}: "
                       f"{L.moe_last_error().decode()}")


# ---------------------------------------------------------------- descriptors
def qformat(bits: int, group: int, mode: int, scale_dtype: int) -> QFormatC:
    return QFormatC(bits, group, mode, scale_dtype)


def layer_desc(hidden, n_experts, top_k, inter, shared_inter, act_dtype,
               router, gate_row, routed, shared) -> LayerDescC:
    """Formats are (bits, group, mode, scale_dtype) tuples or QFormatC."""
    f = lambda q: q if isinstance(q, QFormatC) else QFormatC(*q)
    return LayerDescC(hidden, n_experts, top_k, inter, shared_inter, act_dtype,
                      f(router), f(gate_row), f(routed), f(shared))


def pack_size(desc: LayerDescC) -> int:
    n = C.c_uint64()
    _check(lib().moe_pack_size(C.byref(desc), C.byref(n)), "moe_pack_size")
    return n.value


def _qt(codes, scales, biases, keep):
    arrs = [np.ascontiguousarray(a) if a is not None else None for a in (codes, scales, biases)]
    keep.extend(a for a in arrs if a is not None)
    return QTensorC(*(a.ctypes.data if a is not None else None for a in arrs))


def layer_src(tensors: dict, keep: list) -> LayerSrcC:
    """tensors: name -> (codes, scales, biases) numpy arrays in the canonical layout."""
    return LayerSrcC(*(_qt(*tensors[n], keep) for n in
                       ("router", "gate_row", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")))


def pack_layer_host(desc: LayerDescC, tensors: dict):
    """Host repack into the kernel layout: (uint8 array, LayerC with dev = NULL)."""
    keep = []
    src = layer_src(tensors, keep)
    nbytes = pack_size(desc)
    buf = np.zeros(nbytes, np.uint8)
    out = LayerC()
    _check(lib().moe_pack_layer_host(C.byref(desc), C.byref(src), buf.ctypes.data, nbytes,
                                     C.byref(out)), "moe_pack_layer_host")
    return buf, out


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


@dataclass
class Layer:
    """A packed layer on the device: the LayerC struct and the tensor that owns the bytes."""
    c: LayerC
    buf: object       # torch.uint8 device tensor
    desc: LayerDescC

    @property
    def hidden(self):
        return self.desc.hidden

    @property
    def top_k(self):
        return self.desc.top_k

    @property
    def n_experts(self):
        return self.desc.n_experts


def pack_layer(desc: LayerDescC, tensors: dict, device="cuda", stream=None) -> Layer:
    """Repack on the host and copy to a new device buffer (moe_pack_layer)."""
    import torch
    keep = []
    src = layer_src(tensors, keep)
    nbytes = pack_size(desc)
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    base = buf.data_ptr()
    pad = (-base) % 256
    out = LayerC()
    _check(lib().moe_pack_layer(C.byref(desc), C.byref(src), C.c_void_p(base + pad), nbytes,
                                _stream_ptr(stream), C.byref(out)), "moe_pack_layer")
    return Layer(out, buf, desc)


def workspace_size(desc: LayerDescC, rows: int, grouped) -> int:
    """grouped: False / True (decode / grouped form) or one of MOE_WS_*."""
    n = C.c_uint64()
    _check(lib().moe_workspace_size(C.byref(desc), rows, int(grouped), C.byref(n)),
           "moe_workspace_size")
    return n.value


def new_workspace(layer: "Layer", rows: int, grouped, device="cuda", stream=None):
    """A zero-filled workspace for `rows` rows (route + experts of one layer),
    allocated and cleared on `stream` (default: the current stream), so that
    calls enqueued on that stream find it cleared."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(s):
        return torch.zeros(workspace_size(layer.desc, rows, grouped), dtype=torch.uint8, device=device)


def route_failures(ws, clear=True, stream=None) -> int:
    """moe_route_failures: rows whose decode-router hand-off missed the wait
    bound since the count was last cleared (synchronises `stream`)."""
    n = C.c_uint32()
    _check(lib().moe_route_failures(_ptr(ws), ws.numel() * ws.element_size(), int(clear), C.byref(n),
                                    _stream_ptr(stream)), "moe_route_failures")
    return n.value


def _on(stream):
    """Context in which outputs of a call on `stream` are allocated."""
    import torch
    return torch.cuda.stream(stream) if stream is not None else _nullctx()


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _taps(taps: Optional[dict]):
    """taps: dict of optional device tensors logits/gu/h/e and an optional
    list "events" of torch.cuda.Event (or None) bracketing each kernel."""
    if not taps:
        return None
    t = TapsC()
    for k in ("logits", "gu", "h", "e"):
        v = taps.get(k)
        setattr(t, k, v.data_ptr() if v is not None else None)
    for i, ev in enumerate(taps.get("events") or []):
        t.kernel_events[i] = ev.cuda_event if ev is not None else None
    t.route_wait_limit = int(taps.get("route_wait_limit", 0))
    return C.byref(t)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def route(layer: Layer, x, logit_bias=None, taps=None, out=None, ws=None, stream=None):
    """moe_route: returns (ids int32 [R,k], p fp32 [R,k], shared_gate fp32 [R])."""
    import torch
    R = x.shape[0]
    k = layer.desc.top_k
    with _on(stream):
        if out is None:
            ids = torch.empty((R, k), dtype=torch.int32, device=x.device)
            p = torch.empty((R, k), dtype=torch.float32, device=x.device)
            sg = torch.empty((R,), dtype=torch.float32, device=x.device)
        else:
            ids, p, sg = out
    if ws is None:
        ws = new_workspace(layer, R, R > 16, x.device, stream)
    _check(lib().moe_route(C.byref(layer.c), _ptr(x), R, _ptr(logit_bias), _ptr(ids), _ptr(p),
                           _ptr(sg), _ptr(ws), ws.numel() * ws.element_size(), _taps(taps),
                           _stream_ptr(stream)), "moe_route")
    return ids, p, sg


def experts(layer: Layer, x, ids, p, sg, grouped: bool, ws=None, taps=None, y=None,
            stream=None):
    """moe_experts_decode (grouped=False) or moe_experts_grouped: returns y fp32 [R,H]."""
    import torch
    R = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((R, layer.desc.hidden), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(layer, R, grouped, x.device, stream)
    fn = lib().moe_experts_grouped if grouped else lib().moe_experts_decode
    _check(fn(C.byref(layer.c), _ptr(x), R, _ptr(ids), _ptr(p), _ptr(sg), _ptr(y), _ptr(ws),
              ws.numel() * ws.element_size(), _taps(taps), _stream_ptr(stream)),
           "moe_experts_grouped" if grouped else "moe_experts_decode")
    return y


def forward_windows(layer: Layer, x, logit_bias=None, ws=None, out=None, y=None, stream=None):
    """moe_forward_windows: route + decode experts in windows of 16 rows;
    returns (ids, p, shared_gate, y), each row bit-identical to its one-row step."""
    import torch
    R = x.shape[0]
    k = layer.desc.top_k
    with _on(stream):
        if out is None:
            ids = torch.empty((R, k), dtype=torch.int32, device=x.device)
            p = torch.empty((R, k), dtype=torch.float32, device=x.device)
            sg = torch.empty((R,), dtype=torch.float32, device=x.device)
        else:
            ids, p, sg = out
        if y is None:
            y = torch.empty((R, layer.desc.hidden), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(layer, min(R, 16), False, x.device, stream)
    _check(lib().moe_forward_windows(C.byref(layer.c), _ptr(x), R, _ptr(logit_bias), _ptr(ids), _ptr(p),
                                     _ptr(sg), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream_ptr(stream)), "moe_forward_windows")
    return ids, p, sg, y


def forward_exact(layer: Layer, x, logit_bias=None, ws=None, out=None, y=None, taps=None, stream=None):
    """moe_forward_exact: the chunk with the decode step's bits for every row
    (sorted into expert blocks); returns (ids, p, shared_gate, y)."""
    import torch
    R = x.shape[0]
    k = layer.desc.top_k
    with _on(stream):
        if out is None:
            ids = torch.empty((R, k), dtype=torch.int32, device=x.device)
            p = torch.empty((R, k), dtype=torch.float32, device=x.device)
            sg = torch.empty((R,), dtype=torch.float32, device=x.device)
        else:
            ids, p, sg = out
        if y is None:
            y = torch.empty((R, layer.desc.hidden), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(layer, R, MOE_WS_EXACT, x.device, stream)
    _check(lib().moe_forward_exact(C.byref(layer.c), _ptr(x), R, _ptr(logit_bias), _ptr(ids), _ptr(p),
                                   _ptr(sg), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _taps(taps),
                                   _stream_ptr(stream)), "moe_forward_exact")
    return ids, p, sg, y


def forward_windows_noalloc(layer: Layer, x, logit_bias=None, out=None, y=None, stream=None):
    """moe_forward_windows_noalloc: as forward_windows, with the library's
    fixed device array as the workspace (the call allocates no device
    memory); returns (ids, p, shared_gate, y)."""
    import torch
    R = x.shape[0]
    k = layer.desc.top_k
    with _on(stream):
        if out is None:
            ids = torch.empty((R, k), dtype=torch.int32, device=x.device)
            p = torch.empty((R, k), dtype=torch.float32, device=x.device)
            sg = torch.empty((R,), dtype=torch.float32, device=x.device)
        else:
            ids, p, sg = out
        if y is None:
            y = torch.empty((R, layer.desc.hidden), dtype=torch.float32, device=x.device)
    _check(lib().moe_forward_windows_noalloc(C.byref(layer.c), _ptr(x), R, _ptr(logit_bias), _ptr(ids),
                                             _ptr(p), _ptr(sg), _ptr(y), _stream_ptr(stream)),
           "moe_forward_windows_noalloc")
    return ids, p, sg, y


def experts_decode(layer, x, ids, p, sg, **kw):
    return experts(layer, x, ids, p, sg, False, **kw)


def experts_grouped(layer, x, ids, p, sg, **kw):
    return experts(layer, x, ids, p, sg, True, **kw)
