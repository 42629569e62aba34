"""fp64 CPU oracle for the quantized MoE expert forward (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. Nothing in the GPU library imports it.

Inputs arrive in the canonical layout (codes ``uint8 [rows, cols]``, scale and
bias ``uint16`` bf16 bit patterns ``[rows, cols // group]``); any object with
``codes``, ``scale``, ``bias`` and ``group`` attributes is accepted. Dense
inputs are converted to fp64 exactly (fp32 -> fp64). Every function below is the
plain definition of one step of the method; ``oracle.c`` gives the passages of
the Flash-MoE pages each one follows.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: exact rational brute force, closed forms, algebraic identities, and an
independent library GEMV.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
EPS_RMS = 1e-6


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", os.path.join(_HERE, "oracle.c"), "-o", _SO, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed")


class _QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        i32, vp, dbl = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.orc_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_bf16.restype = dbl
        lib.orc_dequant.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        lib.orc_qmatvec.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        lib.orc_silu.argtypes = [dbl]
        lib.orc_silu.restype = dbl
        lib.orc_sigmoid.argtypes = [dbl]
        lib.orc_sigmoid.restype = dbl
        lib.orc_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        lib.orc_router.argtypes = [i32, i32, vp, vp, vp]
        lib.orc_route.argtypes = [i32, i32, vp, vp, vp, vp]
        lib.orc_shared_gate.argtypes = [i32, vp, vp]
        lib.orc_shared_gate.restype = dbl
        lib.orc_moe_layer.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_rms_scale.argtypes = [i32, vp, dbl, vp]
        lib.orc_set_threads.argtypes = [i32]
        lib.orc_set_threads.restype = None
        lib.orc_get_threads.argtypes = []
        lib.orc_get_threads.restype = i32
        for f in ("orc_dequant", "orc_qmatvec", "orc_expert", "orc_router", "orc_route",
                  "orc_moe_layer", "orc_rms_scale"):
            getattr(lib, f).restype = i32
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} failed with code {rc}")


def _qm(q):
    codes = _c(q.codes, np.uint8)
    scale = _c(q.scale, np.uint16)
    bias = _c(q.bias, np.uint16)
    keep = (codes, scale, bias)
    return _QMat(codes.ctypes.data, scale.ctypes.data, bias.ctypes.data), keep


def set_threads(n: int) -> None:
    """Threads for the row-parallel loops; results are bitwise independent of it."""
    _L().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_L().orc_get_threads())


# ----------------------------------------------------------------------------- steps

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore"):
        return f.astype(np.float64)


def dequant(q) -> np.ndarray:
    """W = code * scale + bias per group, fp64 ``[rows, cols]`` (exact)."""
    codes = _c(q.codes, np.uint8)
    rows, cols = codes.shape
    W = np.empty((rows, cols), dtype=np.float64)
    scale, bias = _c(q.scale, np.uint16), _c(q.bias, np.uint16)
    _check(_L().orc_dequant(rows, cols, q.group, codes.ctypes.data, scale.ctypes.data,
                            bias.ctypes.data, W.ctypes.data), "orc_dequant")
    return W


def qmatvec(q, x) -> np.ndarray:
    """y = dequant(q) @ x in fp64, ascending column order. x: ``[cols]`` or ``[B, cols]``."""
    codes = _c(q.codes, np.uint8)
    rows, cols = codes.shape
    scale, bias = _c(q.scale, np.uint16), _c(q.bias, np.uint16)
    xs = np.atleast_2d(np.asarray(x, dtype=np.float64))
    out = np.empty((xs.shape[0], rows), dtype=np.float64)
    for t in range(xs.shape[0]):
        xt = _c(xs[t], np.float64)
        yt = np.empty(rows, dtype=np.float64)
        _check(_L().orc_qmatvec(rows, cols, q.group, codes.ctypes.data, scale.ctypes.data,
                                bias.ctypes.data, xt.ctypes.data, yt.ctypes.data), "orc_qmatvec")
        out[t] = yt
    return out[0] if np.ndim(x) == 1 else out


def silu(z: float) -> float:
    return float(_L().orc_silu(float(z)))


def sigmoid(z: float) -> float:
    return float(_L().orc_sigmoid(float(z)))


def expert(e: dict, x):
    """SwiGLU expert on one token: returns (h [inter], out [hidden]) in fp64."""
    xs = _c(x, np.float64)
    hidden = xs.shape[0]
    inter = e["gate"].codes.shape[0]
    qs = [_qm(e[k]) for k in ("gate", "up", "down")]
    h = np.empty(inter, dtype=np.float64)
    out = np.empty(hidden, dtype=np.float64)
    _check(_L().orc_expert(hidden, inter, e["gate"].group, ctypes.byref(qs[0][0]), ctypes.byref(qs[1][0]),
                           ctypes.byref(qs[2][0]), xs.ctypes.data, h.ctypes.data, out.ctypes.data),
           "orc_expert")
    return h, out


def router_logits(R, x) -> np.ndarray:
    Rc = _c(R, np.float32)
    xs = _c(x, np.float64)
    logits = np.empty(Rc.shape[0], dtype=np.float64)
    _check(_L().orc_router(Rc.shape[0], Rc.shape[1], Rc.ctypes.data, xs.ctypes.data, logits.ctypes.data),
           "orc_router")
    return logits


def route(logits, k: int):
    """softmax -> top-k (probability descending, lower index on exact ties) -> renormalise.
    Returns (idx int32 [k], w fp64 [k], p fp64 [n])."""
    lg = _c(logits, np.float64)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    p = np.empty(lg.shape[0], dtype=np.float64)
    _check(_L().orc_route(lg.shape[0], k, lg.ctypes.data, idx.ctypes.data, w.ctypes.data, p.ctypes.data),
           "orc_route")
    return idx, w, p


def shared_gate(g, x) -> float:
    gc = _c(g, np.float32)
    xs = _c(x, np.float64)
    return float(_L().orc_shared_gate(gc.shape[0], gc.ctypes.data, xs.ctypes.data))


def moe_layer(R, g, experts, shared: dict, x, residual, k: int):
    """One MoE layer for one token.

    ``experts`` maps expert index -> expert dict (only the chosen ones are needed).
    Returns (out fp64 [hidden], idx int32 [k], w fp64 [k], sigma).
    Raises KeyError naming the missing expert if a chosen expert was not supplied.
    """
    Rc = _c(R, np.float32)
    gc = _c(g, np.float32)
    n_exp, hidden = Rc.shape
    inter = shared["gate"].codes.shape[0]
    group = shared["gate"].group
    arr = (_QMat * (3 * n_exp))()
    keep = []
    for e, ex in experts.items():
        for j, key in enumerate(("gate", "up", "down")):
            qm, kp = _qm(ex[key])
            keep.append(kp)
            arr[3 * e + j] = qm
    sh = (_QMat * 3)()
    for j, key in enumerate(("gate", "up", "down")):
        qm, kp = _qm(shared[key])
        keep.append(kp)
        sh[j] = qm
    xs = _c(x, np.float64)
    rs = _c(residual, np.float64)
    out = np.empty(hidden, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    sig = ctypes.c_double(0.0)
    rc = _L().orc_moe_layer(hidden, inter, group, n_exp, k, Rc.ctypes.data, gc.ctypes.data, arr, sh,
                            xs.ctypes.data, rs.ctypes.data, out.ctypes.data, idx.ctypes.data,
                            w.ctypes.data, ctypes.byref(sig))
    if rc == -2:
        missing = [int(i) for i in idx if int(i) not in experts]
        raise KeyError(missing)
    _check(rc, "orc_moe_layer")
    return out, idx, w, sig.value


def rms_scale(h, eps: float = EPS_RMS) -> np.ndarray:
    hs = _c(h, np.float64)
    x = np.empty_like(hs)
    _check(_L().orc_rms_scale(hs.shape[0], hs.ctypes.data, eps, x.ctypes.data), "orc_rms_scale")
    return x
