"""Python binding of libfmoe, the quantized MoE expert forward for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels
of ``libfmoe.so`` behind the C ABI declared in ``include/fmoe.h``. The functions
keep the C names. Device arrays are torch tensors on the GPU (torch provides
device memory and streams); the stream defaults to torch's current stream.
There is no CPU fallback: if the library is not built, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch  # loaded first so that libfmoe binds to the HIP runtime torch uses

from . import buildlib as _buildlib

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfmoe.so")

GROUP = 64
MAX_TOPK = 16
MAX_TOKENS = 256
MAX_EXPERTS = 1024

STATUS = {
    0: "FMOE_OK", 1: "FMOE_ERR_NULL", 2: "FMOE_ERR_SHAPE", 3: "FMOE_ERR_ALIGN", 4: "FMOE_ERR_BITS",
    5: "FMOE_ERR_ROUTING", 6: "FMOE_ERR_BATCH", 7: "FMOE_ERR_WORKSPACE", 8: "FMOE_ERR_LAUNCH",
    9: "FMOE_ERR_ALIAS",
}


class FmoeError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = lib().fmoe_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


class fmoe_qmat(ctypes.Structure):
    _fields_ = [("blob", ctypes.c_void_p), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32)]


class fmoe_expert(ctypes.Structure):
    _fields_ = [("blob", ctypes.c_void_p), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32)]


class fmoe_layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p), ("bank", ctypes.c_void_p),
                ("shared", ctypes.c_void_p), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32)]


_lib = None

_SIGS = {
    "fmoe_qmat_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "fmoe_expert_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "fmoe_expert_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fmoe_expert)]),
    "fmoe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fmoe_layer), ctypes.c_int]),
    "fmoe_stack_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fmoe_layer), ctypes.c_int]),
    "fmoe_pack_qmat": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4),
    "fmoe_unpack_qmat": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4),
    "fmoe_pack_expert": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4),
    "fmoe_unpack_expert": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4),
    "fmoe_pack_qmat_device": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 5),
    "fmoe_pack_expert_device": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.c_void_p] * 5),
    "fmoe_q4_matvec": (ctypes.c_int, [ctypes.POINTER(fmoe_qmat)] + [ctypes.c_void_p] * 3),
    "fmoe_q2_matvec": (ctypes.c_int, [ctypes.POINTER(fmoe_qmat)] + [ctypes.c_void_p] * 3),
    "fmoe_qmatvec_form": (ctypes.c_int, [ctypes.POINTER(fmoe_qmat), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]),
    "fmoe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(fmoe_expert), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fmoe_expert_ffn_form": (ctypes.c_int, [ctypes.POINTER(fmoe_expert), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "fmoe_moe_layer_form": (ctypes.c_int, [ctypes.POINTER(fmoe_layer)] + [ctypes.c_void_p] * 6 +
                            [ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "fmoe_moe_layer": (ctypes.c_int, [ctypes.POINTER(fmoe_layer), ctypes.c_int] + [ctypes.c_void_p] * 6 +
                       [ctypes.c_size_t, ctypes.c_void_p]),
    "fmoe_moe_layer_phases": (ctypes.c_int, [ctypes.POINTER(fmoe_layer), ctypes.c_int] + [ctypes.c_void_p] * 6 +
                              [ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "fmoe_moe_layer_noalloc": (ctypes.c_int, [ctypes.POINTER(fmoe_layer), ctypes.c_int] + [ctypes.c_void_p] * 6),
    "fmoe_cache_device_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "fmoe_cache_create": (ctypes.c_int, [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_size_t,
                                                              ctypes.POINTER(ctypes.c_void_p)]),
    "fmoe_cache_destroy": (None, [ctypes.c_void_p]),
    "fmoe_cache_get_stats": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.POINTER(ctypes.c_int64)] * 4),
    "fmoe_cache_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "fmoe_tiered_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fmoe_layer), ctypes.c_int]),
    "fmoe_moe_layer_tiered": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(fmoe_layer), ctypes.c_int] +
                              [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "fmoe_moe_layer_tiered_device": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(fmoe_layer),
                                                    ctypes.c_int] + [ctypes.c_void_p] * 6 +
                                     [ctypes.c_size_t, ctypes.c_void_p]),
    "fmoe_rms_scale": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_void_p]),
    "fmoe_moe_stack": (ctypes.c_int, [ctypes.POINTER(fmoe_layer), ctypes.c_int, ctypes.c_int] +
                       [ctypes.c_void_p] * 5 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                                ctypes.c_void_p]),
    "fmoe_moe_stack_trace": (ctypes.c_int, [ctypes.POINTER(fmoe_layer), ctypes.c_int, ctypes.c_int] +
                             [ctypes.c_void_p] * 2 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "fmoe_read_xor": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "fmoe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fmoe_version": (ctypes.c_int, []),
}


def lib():
    """The loaded libfmoe (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ok(status: int, where: str) -> None:
    if status != 0:
        raise FmoeError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous float32 CUDA tensor")
    return t


# ----------------------------------------------------------------------------- handles

@dataclass
class QMat:
    """A packed quantized matrix resident on the device."""
    blob: object  # uint8 CUDA tensor or raw device pointer
    rows: int
    cols: int
    bits: int
    group: int = GROUP

    def c(self) -> fmoe_qmat:
        return fmoe_qmat(_ptr(self.blob), self.rows, self.cols, self.bits, self.group)


@dataclass
class Expert:
    """A packed SwiGLU expert resident on the device."""
    blob: object
    hidden: int
    inter: int
    bits: int
    group: int = GROUP

    def c(self) -> fmoe_expert:
        return fmoe_expert(_ptr(self.blob), self.hidden, self.inter, self.bits, self.group)


@dataclass
class Layer:
    """One MoE layer: router, expert bank, optional shared expert and its gate vector."""
    router: object
    shared_gate: object
    bank: object
    shared: object
    n_experts: int
    top_k: int
    hidden: int
    inter: int
    bits: int
    group: int = GROUP

    def c(self) -> fmoe_layer:
        return fmoe_layer(_ptr(self.router), _ptr(self.shared_gate), _ptr(self.bank), _ptr(self.shared),
                          self.n_experts, self.top_k, self.hidden, self.inter, self.bits, self.group)


# ----------------------------------------------------------------------------- sizes

def fmoe_qmat_bytes(bits: int, rows: int, cols: int, group: int = GROUP) -> int:
    return int(lib().fmoe_qmat_bytes(bits, rows, cols, group))


def fmoe_expert_bytes(bits: int, hidden: int, inter: int, group: int = GROUP) -> int:
    return int(lib().fmoe_expert_bytes(bits, hidden, inter, group))


def fmoe_expert_workspace_bytes(E: Expert) -> int:
    return int(lib().fmoe_expert_workspace_bytes(ctypes.byref(E.c())))


def fmoe_workspace_bytes(L: Layer, n_tokens: int) -> int:
    return int(lib().fmoe_workspace_bytes(ctypes.byref(L.c()), n_tokens))


def fmoe_stack_workspace_bytes(L: Layer, n_tokens: int) -> int:
    return int(lib().fmoe_stack_workspace_bytes(ctypes.byref(L.c()), n_tokens))


# ----------------------------------------------------------------------------- packing (host)

def _canon(codes, scale, bias):
    return (np.ascontiguousarray(codes, dtype=np.uint8), np.ascontiguousarray(scale, dtype=np.uint16),
            np.ascontiguousarray(bias, dtype=np.uint16))


def fmoe_pack_qmat(bits: int, codes, scale, bias, group: int = GROUP) -> np.ndarray:
    """Canonical host arrays -> packed host blob (uint8)."""
    c, s, b = _canon(codes, scale, bias)
    rows, cols = c.shape
    n = fmoe_qmat_bytes(bits, rows, cols, group)
    out = np.empty(max(n, 1), dtype=np.uint8)
    _ok(lib().fmoe_pack_qmat(bits, rows, cols, group, c.ctypes.data, s.ctypes.data, b.ctypes.data,
                             out.ctypes.data), "fmoe_pack_qmat")
    return out


def fmoe_unpack_qmat(bits: int, rows: int, cols: int, blob, group: int = GROUP):
    bl = np.ascontiguousarray(blob, dtype=np.uint8)
    c = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // group), np.uint16)
    b = np.empty((rows, cols // group), np.uint16)
    _ok(lib().fmoe_unpack_qmat(bits, rows, cols, group, bl.ctypes.data, c.ctypes.data, s.ctypes.data,
                               b.ctypes.data), "fmoe_unpack_qmat")
    return c, s, b


def _triple(vals, ctype):
    arr = (ctypes.c_void_p * 3)(*[v.ctypes.data if isinstance(v, np.ndarray) else _ptr(v) for v in vals])
    return arr


def fmoe_pack_expert(bits: int, gate, up, down, group: int = GROUP) -> np.ndarray:
    """gate, up, down: (codes, scale, bias) tuples or objects with those attributes."""
    mats = [_canon(*(m if isinstance(m, tuple) else (m.codes, m.scale, m.bias))) for m in (gate, up, down)]
    inter, hidden = mats[0][0].shape
    n = fmoe_expert_bytes(bits, hidden, inter, group)
    out = np.empty(max(n, 1), dtype=np.uint8)
    codes = (ctypes.c_void_p * 3)(*[m[0].ctypes.data for m in mats])
    scale = (ctypes.c_void_p * 3)(*[m[1].ctypes.data for m in mats])
    bias = (ctypes.c_void_p * 3)(*[m[2].ctypes.data for m in mats])
    _ok(lib().fmoe_pack_expert(bits, hidden, inter, group, codes, scale, bias, out.ctypes.data),
        "fmoe_pack_expert")
    return out


def fmoe_unpack_expert(bits: int, hidden: int, inter: int, blob, group: int = GROUP):
    bl = np.ascontiguousarray(blob, dtype=np.uint8)
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    cs = [np.empty(sh, np.uint8) for sh in shapes]
    ss = [np.empty((sh[0], sh[1] // group), np.uint16) for sh in shapes]
    bs = [np.empty((sh[0], sh[1] // group), np.uint16) for sh in shapes]
    codes = (ctypes.c_void_p * 3)(*[a.ctypes.data for a in cs])
    scale = (ctypes.c_void_p * 3)(*[a.ctypes.data for a in ss])
    bias = (ctypes.c_void_p * 3)(*[a.ctypes.data for a in bs])
    _ok(lib().fmoe_unpack_expert(bits, hidden, inter, group, bl.ctypes.data, codes, scale, bias),
        "fmoe_unpack_expert")
    return list(zip(cs, ss, bs))


# ----------------------------------------------------------------------------- packing (device)

def fmoe_pack_qmat_device(bits: int, rows: int, cols: int, codes, scale, bias, blob_out, group: int = GROUP,
                          stream=None) -> None:
    _ok(lib().fmoe_pack_qmat_device(bits, rows, cols, group, _ptr(codes), _ptr(scale), _ptr(bias),
                                    _ptr(blob_out), _stream(stream)), "fmoe_pack_qmat_device")


def fmoe_pack_expert_device(bits: int, hidden: int, inter: int, codes: Sequence, scale: Sequence,
                            bias: Sequence, blob_out, group: int = GROUP, stream=None) -> None:
    c = (ctypes.c_void_p * 3)(*[_ptr(t) for t in codes])
    s = (ctypes.c_void_p * 3)(*[_ptr(t) for t in scale])
    b = (ctypes.c_void_p * 3)(*[_ptr(t) for t in bias])
    _ok(lib().fmoe_pack_expert_device(bits, hidden, inter, group, c, s, b, _ptr(blob_out), _stream(stream)),
        "fmoe_pack_expert_device")


# ----------------------------------------------------------------------------- compute

def fmoe_q4_matvec(W: QMat, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev_f32(x, "x")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _ok(lib().fmoe_q4_matvec(ctypes.byref(W.c()), _ptr(x), _ptr(y), _stream(stream)), "fmoe_q4_matvec")
    return y


def fmoe_q2_matvec(W: QMat, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev_f32(x, "x")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    _ok(lib().fmoe_q2_matvec(ctypes.byref(W.c()), _ptr(x), _ptr(y), _stream(stream)), "fmoe_q2_matvec")
    return y


def fmoe_qmatvec_form(W: QMat, x: torch.Tensor, form: int, y: Optional[torch.Tensor] = None,
                      stream=None, c_qmat=None) -> torch.Tensor:
    """y = W x with the per-weight arithmetic in form 0 (naive), 1 (fma recast),
    2 (group-factored) or 3 (table in LDS); either bit width."""
    _dev_f32(x, "x")
    if y is None:
        y = torch.empty(W.rows, dtype=torch.float32, device=x.device)
    cq = c_qmat if c_qmat is not None else W.c()
    _ok(lib().fmoe_qmatvec_form(ctypes.byref(cq), _ptr(x), _ptr(y), form, _stream(stream)), "fmoe_qmatvec_form")
    return y


def fmoe_expert_ffn(E: Expert, x: torch.Tensor, out: Optional[torch.Tensor] = None, ws=None,
                    stream=None) -> torch.Tensor:
    _dev_f32(x, "x")
    if out is None:
        out = torch.empty(E.hidden, dtype=torch.float32, device=x.device)
    need = fmoe_expert_workspace_bytes(E)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_expert_ffn(ctypes.byref(E.c()), _ptr(x), _ptr(out), _ptr(ws), nbytes, _stream(stream)),
        "fmoe_expert_ffn")
    return out


def fmoe_expert_ffn_form(E: Expert, x: torch.Tensor, form: int, out: Optional[torch.Tensor] = None, ws=None,
                         stream=None, c_expert=None) -> torch.Tensor:
    """fmoe_expert_ffn with the per-weight arithmetic of every projection in form 0 (naive),
    1 (fma recast), 2 (group-factored) or 3 (table in LDS)."""
    _dev_f32(x, "x")
    if out is None:
        out = torch.empty(E.hidden, dtype=torch.float32, device=x.device)
    need = fmoe_expert_workspace_bytes(E)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    ce = c_expert if c_expert is not None else E.c()
    _ok(lib().fmoe_expert_ffn_form(ctypes.byref(ce), _ptr(x), _ptr(out), _ptr(ws), nbytes, form, _stream(stream)),
        "fmoe_expert_ffn_form")
    return out


def fmoe_moe_layer(L: Layer, x: torch.Tensor, residual: torch.Tensor, out: Optional[torch.Tensor] = None,
                   topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None, ws=None,
                   stream=None) -> torch.Tensor:
    """x, residual: [n_tokens, hidden] float32 on the device."""
    _dev_f32(x, "x")
    _dev_f32(residual, "residual")
    n_tokens = x.shape[0] if x.dim() == 2 else 1
    if out is None:
        out = torch.empty_like(residual)
    need = fmoe_workspace_bytes(L, n_tokens)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_moe_layer(ctypes.byref(L.c()), n_tokens, _ptr(x), _ptr(residual), _ptr(out), _ptr(topk_idx),
                             _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)), "fmoe_moe_layer")
    return out


def fmoe_moe_layer_form(L: Layer, x: torch.Tensor, residual: torch.Tensor, form: int,
                        out: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                        topk_w: Optional[torch.Tensor] = None, ws=None, stream=None, c_layer=None) -> torch.Tensor:
    """fmoe_moe_layer for one token (x, residual: [hidden] or [1, hidden]) with the expert
    projections' per-weight arithmetic in form 0 (naive), 1 (fma recast), 2 (group-factored)
    or 3 (table in LDS)."""
    _dev_f32(x, "x")
    _dev_f32(residual, "residual")
    if out is None:
        out = torch.empty_like(residual)
    need = fmoe_workspace_bytes(L, 1)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    cl = c_layer if c_layer is not None else L.c()
    _ok(lib().fmoe_moe_layer_form(ctypes.byref(cl), _ptr(x), _ptr(residual), _ptr(out), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(ws), nbytes, form, _stream(stream)), "fmoe_moe_layer_form")
    return out


def fmoe_moe_layer_phases(L: Layer, x: torch.Tensor, residual: torch.Tensor, out: torch.Tensor, phases: int,
                          ws, topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                          stream=None, c_layer=None) -> None:
    """Enqueue only some of the layer's three kernels (bit mask `phases`); for per-kernel timing."""
    n_tokens = x.shape[0] if x.dim() == 2 else 1
    cl = c_layer if c_layer is not None else L.c()
    nbytes = ws.numel() * ws.element_size()
    _ok(lib().fmoe_moe_layer_phases(ctypes.byref(cl), n_tokens, _ptr(x), _ptr(residual), _ptr(out), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(ws), nbytes, phases, _stream(stream)), "fmoe_moe_layer_phases")


NOALLOC_SCRATCH_BYTES = 4 << 20  # FMOE_NOALLOC_SCRATCH_BYTES


def fmoe_moe_layer_noalloc(L: Layer, x: torch.Tensor, residual: torch.Tensor, out: torch.Tensor,
                           topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """fmoe_moe_layer with the library's static per-GPU workspace: allocates nothing, so
    `out` must be given. Calls that may overlap on one GPU race."""
    _dev_f32(x, "x")
    _dev_f32(residual, "residual")
    _dev_f32(out, "out")
    n_tokens = x.shape[0] if x.dim() == 2 else 1
    _ok(lib().fmoe_moe_layer_noalloc(ctypes.byref(L.c()), n_tokens, _ptr(x), _ptr(residual), _ptr(out),
                                     _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "fmoe_moe_layer_noalloc")
    return out


# ----------------------------------------------------------------------------- host-memory expert tier

def fmoe_cache_device_bytes(bits: int, hidden: int, inter: int, n_experts: int, n_slots: int,
                            group: int = GROUP) -> int:
    return int(lib().fmoe_cache_device_bytes(bits, hidden, inter, group, n_experts, n_slots))


def fmoe_cache_create(bits: int, hidden: int, inter: int, n_experts: int, n_slots: int, device_buf,
                      group: int = GROUP) -> ctypes.c_void_p:
    nbytes = device_buf.numel() * device_buf.element_size() if isinstance(device_buf, torch.Tensor) else 0
    h = ctypes.c_void_p()
    _ok(lib().fmoe_cache_create(bits, hidden, inter, group, n_experts, n_slots, _ptr(device_buf), nbytes,
                                ctypes.byref(h)), "fmoe_cache_create")
    return h


def fmoe_cache_destroy(handle) -> None:
    lib().fmoe_cache_destroy(handle)


def fmoe_cache_get_stats(handle) -> dict:
    v = [ctypes.c_int64() for _ in range(4)]
    _ok(lib().fmoe_cache_get_stats(handle, *[ctypes.byref(x) for x in v]), "fmoe_cache_get_stats")
    return dict(zip(("lookups", "hits", "misses", "bytes_copied"), (x.value for x in v)))


def fmoe_cache_plan(handle, layer: int, experts):
    """The cache's policy step alone (host only): returns (slots, misses) for the
    distinct experts of one call."""
    e = np.ascontiguousarray(experts, dtype=np.int32)
    slots = np.empty(e.size, np.int32)
    miss = np.empty(e.size, np.int32)
    _ok(lib().fmoe_cache_plan(handle, layer, e.ctypes.data, e.size, slots.ctypes.data, miss.ctypes.data),
        "fmoe_cache_plan")
    return slots, miss


class ExpertCache:
    """An HBM cache of n_slots expert blobs for the host-memory expert tier (device
    buffer allocated here with torch; the library owns only host bookkeeping)."""

    def __init__(self, bits: int, hidden: int, inter: int, n_experts: int, n_slots: int, device="cuda"):
        nb = fmoe_cache_device_bytes(bits, hidden, inter, n_experts, n_slots)
        if nb == 0:
            raise FmoeError(2, "fmoe_cache_device_bytes")
        self.buf = torch.empty(nb, dtype=torch.uint8, device=device)
        self.handle = fmoe_cache_create(bits, hidden, inter, n_experts, n_slots, self.buf)

    def stats(self) -> dict:
        return fmoe_cache_get_stats(self.handle)

    def plan(self, layer: int, experts):
        return fmoe_cache_plan(self.handle, layer, experts)

    def close(self) -> None:
        if getattr(self, "handle", None):
            fmoe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fmoe_tiered_workspace_bytes(L: Layer, n_tokens: int) -> int:
    return int(lib().fmoe_tiered_workspace_bytes(ctypes.byref(L.c()), n_tokens))


def fmoe_moe_layer_tiered(cache: ExpertCache, layer: int, L: Layer, x: torch.Tensor, residual: torch.Tensor,
                          out: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                          topk_w: Optional[torch.Tensor] = None, ws=None, stream=None) -> torch.Tensor:
    """One MoE layer whose routed expert bank (L.bank) is in host memory (a pinned CPU
    tensor): the chosen experts go through the HBM cache. Synchronises the stream once."""
    _dev_f32(x, "x")
    _dev_f32(residual, "residual")
    n_tokens = x.shape[0] if x.dim() == 2 else 1
    if out is None:
        out = torch.empty_like(residual)
    need = fmoe_tiered_workspace_bytes(L, n_tokens)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_moe_layer_tiered(cache.handle, layer, ctypes.byref(L.c()), n_tokens, _ptr(x), _ptr(residual),
                                    _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)),
        "fmoe_moe_layer_tiered")
    return out


def fmoe_moe_layer_tiered_device(cache: ExpertCache, layer: int, L: Layer, x: torch.Tensor, residual: torch.Tensor,
                                 out: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                                 topk_w: Optional[torch.Tensor] = None, ws=None, stream=None) -> torch.Tensor:
    """fmoe_moe_layer_tiered with the cache's policy and the copies on the GPU: no host
    synchronisation (L.bank: a pinned CPU tensor)."""
    _dev_f32(x, "x")
    _dev_f32(residual, "residual")
    n_tokens = x.shape[0] if x.dim() == 2 else 1
    if out is None:
        out = torch.empty_like(residual)
    need = fmoe_tiered_workspace_bytes(L, n_tokens)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_moe_layer_tiered_device(cache.handle, layer, ctypes.byref(L.c()), n_tokens, _ptr(x),
                                           _ptr(residual), _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                                           nbytes, _stream(stream)),
        "fmoe_moe_layer_tiered_device")
    return out


def fmoe_rms_scale(h: torch.Tensor, x: Optional[torch.Tensor] = None, eps: float = 1e-6,
                   stream=None) -> torch.Tensor:
    _dev_f32(h, "h")
    if x is None:
        x = torch.empty_like(h)
    n_tokens, hidden = (h.shape[0], h.shape[1]) if h.dim() == 2 else (1, h.shape[0])
    _ok(lib().fmoe_rms_scale(_ptr(h), _ptr(x), n_tokens, hidden, eps, _stream(stream)), "fmoe_rms_scale")
    return x


def fmoe_moe_stack(layers: Sequence[Layer], h0: torch.Tensor, h_out: Optional[torch.Tensor] = None,
                   h_all: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None, eps: float = 1e-6, ws=None, stream=None,
                   c_layers=None) -> torch.Tensor:
    """h0: [n_tokens, hidden]. `c_layers` may pass a prebuilt ctypes array of fmoe_layer."""
    _dev_f32(h0, "h0")
    n_tokens = h0.shape[0]
    if h_out is None:
        h_out = torch.empty_like(h0)
    arr = c_layers if c_layers is not None else (fmoe_layer * len(layers))(*[L.c() for L in layers])
    need = int(lib().fmoe_stack_workspace_bytes(ctypes.byref(arr[0]), n_tokens))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=h0.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_moe_stack(arr, len(arr), n_tokens, _ptr(h0), _ptr(h_out), _ptr(h_all), _ptr(topk_idx),
                             _ptr(topk_w), eps, _ptr(ws), nbytes, _stream(stream)), "fmoe_moe_stack")
    return h_out


TRACE_BLOCKS, TRACE_SLOTS = 4096, 8  # FMOE_TRACE_BLOCKS, FMOE_TRACE_SLOTS


def fmoe_moe_stack_trace(layers: Sequence[Layer], h0: torch.Tensor, trace: torch.Tensor, trace_layer: int,
                         h_out: Optional[torch.Tensor] = None, eps: float = 1e-6, ws=None, stream=None,
                         c_layers=None) -> torch.Tensor:
    """fmoe_moe_stack with device-clock stamps of layer `trace_layer`'s
    kernels in `trace` (int64 [3, TRACE_BLOCKS, TRACE_SLOTS] on the device, zeroed by the caller)."""
    _dev_f32(h0, "h0")
    if trace.dtype != torch.int64 or trace.numel() < 3 * TRACE_BLOCKS * TRACE_SLOTS or not trace.is_cuda:
        raise ValueError("trace: int64 device tensor of 3 * TRACE_BLOCKS * TRACE_SLOTS entries")
    n_tokens = h0.shape[0]
    if h_out is None:
        h_out = torch.empty_like(h0)
    arr = c_layers if c_layers is not None else (fmoe_layer * len(layers))(*[L.c() for L in layers])
    need = int(lib().fmoe_stack_workspace_bytes(ctypes.byref(arr[0]), n_tokens))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=h0.device)
    nbytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need
    _ok(lib().fmoe_moe_stack_trace(arr, len(arr), n_tokens, _ptr(h0), _ptr(h_out), eps, _ptr(ws), nbytes,
                                   _ptr(trace), trace_layer, _stream(stream)), "fmoe_moe_stack_trace")
    return h_out


def fmoe_read_xor(buf: Optional[torch.Tensor], out: torch.Tensor, nbytes: Optional[int] = None,
                  stream=None) -> None:
    """out (int32 [1] on the device) ^= XOR of the 32-bit words of the first nbytes
    (default: all) bytes of buf; buf None or nbytes 0: an empty kernel."""
    if nbytes is None:
        nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    _ok(lib().fmoe_read_xor(_ptr(buf), nbytes, _ptr(out), _stream(stream)), "fmoe_read_xor")


def fmoe_status_string(status: int) -> str:
    return lib().fmoe_status_string(status).decode()


def fmoe_version() -> int:
    return int(lib().fmoe_version())


build = _buildlib.build
